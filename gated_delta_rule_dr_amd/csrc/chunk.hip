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
// Per chunk, with incoming state S and chunk-local cumulative log-decay g_t (per channel, or
// one per head):
//   K+ = k e^{g}, Q+ = q e^{g}, K^end = k e^{g_C - g}, U^end = (e * k) e^{g_C - g}
//   A_kk = strict_lower(k_t . k_i e^{g_t - g_i})  A_ku = strict_lower(k_t . u_i e^{g_t - g_i})
//   A_qk = lower(q_t . k_i e^{g_t - g_i})          A_qu = lower(q_t . u_i e^{g_t - g_i})
//   X_K = K+ S,  X_Q = Q+ S
// symmetric gates (one beta for erase and write):
//   T = (I + Diag(beta) A_kk)^{-1},  delta = T Diag(beta) (V - X_K)
//   O = X_Q + A_qk delta,            S <- Diag(e^{g_C}) S + K^end^T delta
// general gates (erase e, write w; Vt = w * v):
//   T = (I + A_ku)^{-1},  M = T (X_K + A_kk Vt)
//   O = X_Q + A_qk Vt - A_qu M,  S <- Diag(e^{g_C}) S + K^end^T Vt - U^end^T M
//
// Range.  The method allows any decay a in (0, 1) ("Gated DeltaNet-2", gate table; "FG2-GDN",
// section 2, update rule), so no factor that scales an fp16 operand may grow with the decay:
// every one is e^{x} with x <= 0 -- the scan's tiles are referenced at the chunk start, the
// Gram matrices' off-diagonal 16-token blocks at their block boundaries -- except for the
// diagonal blocks' midpoint split, which is taken only where it stays within e^{+-6}.  A
// factor then underflows only where the term it scales is negligible.
//
// Two kernels.  The prep (one workgroup per chunk, all chunks of all heads in parallel) writes
// everything that does not depend on the state into a per-chunk packet in the caller's
// workspace: T (the only factor that needs a serial algorithm), the Gram matrices, the gate
// factors and, unless the decay is one scalar per token, the decayed fp16 operand tiles K+, Q+,
// K^end (and U^end).  The scan then walks the chunks of one (b, h, value slice) in order,
// carrying the fp32 state in registers; per chunk it copies the packet into LDS and runs only
// the state-dependent products, so no exponential, prefix sum or format conversion is repeated
// by the value slices of a head.  With a scalar decay the packet holds no decayed tiles: it
// carries the plain k and q, and the scan applies the per-token factors e^{g_t} and
// e^{g_C - g_t} to product rows instead.
//
// FG2-GDN's per-channel rate beta runs the symmetric kernels on the scaled pair
// (sqrt(beta) k, sqrt(beta) v) with a unit gate: the prep scales k as it loads it and writes the
// scaled values into the packet, from where the scan copies its value slice.  Packed sequences
// of different lengths run the same kernels over tables of their chunks (prep) and sequences
// (scan), written into the workspace by a set-up kernel.
//
// Products use v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation).  Gram tiles are
// computed transposed (A^T = K Q^T) so that each lane owns four consecutive columns of one row
// of A and stores them with one vector write.

#include "chunk_layout.h"
#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

// The same as fp16 into a chunk's state checkpoint at dst ([dv / 16][dk][16]: 16-column tiles).
// The lane holds rows 4 lg + 0..3 of column l16 of each 16 x 16 tile; after the quad transpose it
// holds four consecutive columns of one row and stores them as one 8-byte piece, so that each wave
// writes 16 whole rows of a tile, 512 contiguous bytes.
template <int NCT>
__device__ __forceinline__ void store_state_h(void* dst, int j0, const f32x4 (&S)[NCT]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lg = lane >> 4;
  const int b = l16 & 3, a4 = l16 & 12;
  _Float16* d = static_cast<_Float16*>(dst);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
    *reinterpret_cast<half4v*>(d + ((j0 >> 4) + ct) * (D * 16) + (16 * wave + 4 * lg + b) * 16 + a4) =
        cvt4(quad_transpose(S[ct]));
}

// Halves per chunk of the one-gate A_kk side buffer (the six stored 16 x 32 blocks).
constexpr int64_t kAkkHalves = 6 * 512;

// Rows t0 .. t0 + 3 of column j of a per-chunk fp16 [D / 16][C][16] matrix (packet index pkt)
// from an accumulator tile's four values (j = j_tile + l16): after the quad transpose the lane
// stores four consecutive columns of row t0 + l16 % 4 as one 8-byte piece.
__device__ __forceinline__ void store_rows(void* base, int64_t pkt, int t0, int j, f32x4 x) {
  const int b = threadIdx.x & 3, jb = j - b;
  _Float16* dst = static_cast<_Float16*>(base) + pkt * C * D + (jb >> 4) * (C * 16) + (t0 + b) * 16 + (jb & 15);
  *reinterpret_cast<half4v*>(dst) = cvt4(quad_transpose(x));
}



// The sequence of a scan workgroup (bh = sequence * H + h): the row of its first token, its
// tokens and chunks, and the packet index of its first chunk for head h.  A dense batch stores
// the packets of (b, h) one after another; packed sequences take their place from the table.
struct SeqRef {
  int64_t tok0;
  int len, nch;
  int64_t pkt0;
};
__device__ __forceinline__ SeqRef seq_ref(const Problem& p, int bh, int h) {
  SeqRef r;
  if (p.seqs) {
    const int4 e = p.seqs[bh / p.H];
    r.tok0 = e.x;
    r.len = e.y;
    r.nch = e.w;
    r.pkt0 = int64_t(e.z) + int64_t(h) * e.w;
  } else {
    r.nch = (p.T + C - 1) / C;
    r.tok0 = int64_t(bh / p.H) * p.T;
    r.len = p.T;
    r.pkt0 = int64_t(bh) * r.nch;
  }
  return r;
}

// The (sequence * H + head, value slice) of a scan workgroup.  A dense batch maps blockIdx
// directly; packed sequences take the sequences longest first (the workgroups start in the
// order of their linear index), all heads and slices of one sequence together.
struct WgRef {
  int bh, slice;
};
__device__ __forceinline__ WgRef wg_ref(const Problem& p) {
  WgRef r{int(blockIdx.x), int(blockIdx.y)};
  if (p.order) {
    const int per = p.H * int(gridDim.y);
    const int w = int(blockIdx.x) + int(gridDim.x) * int(blockIdx.y);
    const int rank = w / per, rem = w - rank * per;
    r.slice = rem / p.H;
    r.bh = p.order[rank] * p.H + (rem - r.slice * p.H);
  }
  return r;
}

// A sequence without tokens: S_T = S0 (zeros without S0) on this workgroup's value columns.
__device__ void pass_state(const Problem& p, int bh, int j0, int ncols) {
  if (!p.S_T) return;
  for (int i = threadIdx.x; i < D * ncols; i += blockDim.x) {
    const int d = i / ncols, j = j0 + i % ncols;
    const int64_t x = (int64_t(bh) * D + d) * D + j;
    p.S_T[x] = p.S0 ? p.S0[x] : 0.f;
  }
}

// This wave's part of a scan's fp32 state tiles (rows 16 w + 4 lg + r, columns j0 + 16 ct + l16)
// into the [dk][dv] matrix at dst.
template <int NCT>
__device__ __forceinline__ void store_state(float* dst, int j0, const f32x4 (&S)[NCT]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * wave + 4 * lg + r) * D + j0 + 16 * ct + l16] = S[ct][r];
}


// The solve factor T (fp16 in LDS, row stride CS, zero upper triangle) into the six stored
// 16 x 32 blocks of the packet's first matrix.
__device__ __forceinline__ void write_tri_t(char* mat, const _Float16* TH, int tid) {
  _Float16* wsc = reinterpret_cast<_Float16*>(mat);
  const int t = tid >> 2, c0 = (tid & 3) * 16;
  if (c0 < 32 || t >= 32) {  // the blocks that hold nonzeros
    *reinterpret_cast<uint4*>(wsc + tri_pos(t, c0)) = *reinterpret_cast<const uint4*>(TH + t * CS + c0);
    *reinterpret_cast<uint4*>(wsc + tri_pos(t, c0 + 8)) = *reinterpret_cast<const uint4*>(TH + t * CS + c0 + 8);
  }
}

// T = (I + A)^{-1} for the strictly lower-triangular fp32 A in AF (row stride AFS), into TH
// (fp16, zero upper triangle, which the caller has cleared).  Ends with a barrier.
__device__ __forceinline__ void solve_t(const float* AF, _Float16* TH, int tid) {
  // (the lane index through an empty asm: the identity's entries (r == col) and the lane's LDS
  // addresses are then formed here, in every call, instead of being hoisted out of a caller's
  // chunk loop as invariants that spill, each reload of which waits for every outstanding
  // packet store)
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const int wave = tid >> 6, l16 = lane & 15, lg = lane >> 4;
    // Diagonal 16x16 blocks: fp32 forward substitution, one lane per (block, column).
    if (wave == 0) {
      const int bl = lg, col = l16;
      const float* Ab = AF + (16 * bl) * AFS + 16 * bl;
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
      for (int r = 0; r < 16; ++r) TH[(16 * bl + r) * CS + 16 * bl + col] = (_Float16)x[r];
    }
    lds_barrier();

    // Off-diagonal blocks, level by level: T_JI = -T_JJ sum_{K=I}^{J-1} A_JK T_KI.
#pragma unroll
    for (int Jb = 1; Jb < 4; ++Jb) {
      if (wave < Jb) {
        const int Ib = wave;
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
        for (int Kb = Ib; Kb < Jb; ++Kb) {
          const float4 a4 = *reinterpret_cast<const float4*>(AF + (16 * Jb + l16) * AFS + 16 * Kb + 4 * lg);
          half4v a, bt;
          a[0] = (_Float16)a4.x; a[1] = (_Float16)a4.y; a[2] = (_Float16)a4.z; a[3] = (_Float16)a4.w;
#pragma unroll
          for (int i = 0; i < 4; ++i) bt[i] = TH[(16 * Kb + 4 * lg + i) * CS + 16 * Ib + l16];
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
      lds_barrier();
    }
}

template <int N>
struct IntTag {
  static constexpr int value = N;
};

// ------------------------------------------------------------------------------------------
// Prep, per-head decay with one per-head erase/write gate (scalar-gate Gated DeltaNet; FG2's
// rate with a per-head decay).  Persistent: each workgroup walks every grid-th chunk with the
// next chunk's inputs in flight.  The decay is one scalar per token, so the Gram products run on
// the plain k and q tiles and take the decay between token i and token t >= i per element,
// e^{g_t - g_i} <= 1, in fp32.  The packet carries plain k and q and the scan's per-token
// factors relative to the chunk start, e^{g_t} (rows of K S and Q S) and e^{g_C - g_t} (rows of
// the update's delta), so every factor is at most one whatever the decay.
// ------------------------------------------------------------------------------------------
template <bool FG2>
__global__ __launch_bounds__(kThreads, 1) void chunk_prep_scalar_kernel(Problem p, char* __restrict__ ws,
                                                                        int nchunks, int64_t nblk) {
  // Packed sequences: the work items are (chunk, head) pairs over the chunk table.
  if (p.chunks) nblk = int64_t(p.H) * *p.nchunks_total;
  using PK = Packet<false, false, FG2>;
  __shared__ __attribute__((aligned(16))) _Float16 KP[C * KS];  // k
  __shared__ __attribute__((aligned(16))) _Float16 QP[C * KS];  // q
  __shared__ __attribute__((aligned(16))) float AF[C * AFS];    // fp32 matrix of the solve
  __shared__ __attribute__((aligned(16))) _Float16 TH[C * CS];
  __shared__ float GB[C];
  __shared__ float GSC[C];  // chunk-local cumulative log-decay per token

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  const int d8 = tid & 15, tg = tid >> 4;
  const int H = p.H;
  const gptr<const uint16_t> kin = opaque_gptr(static_cast<const uint16_t*>(p.k));
  const gptr<const uint16_t> qin = opaque_gptr(static_cast<const uint16_t*>(p.q));
  const gptr<const float> ldin = opaque_gptr(p.log_decay);
  const gptr<const float> erin = opaque_gptr(p.erase);

  // Inputs of one chunk in registers: thread (token quad tg, channel octet d8) holds tokens
  // 4 tg + r, channels 8 d8 .. + 7; threads < 64 hold token tid's per-head gates.  Tokens past
  // the end load token T - 1 (zeroed where they are used), so every load is unconditional.
  struct In {
    uint4 kr[4], qr[4];
    float lds, gb;
  };
  // Work item blk: a dense batch walks (b, h, chunk) with packet index blk; packed sequences
  // walk (chunk, head) over the chunk table.  Work items number fewer than 2^31 (one packet
  // each, and the packets fit in device memory), so the index arithmetic is 32-bit.
  auto chunk_ref = [&](int64_t blk) { return chunk_ref_of(p, blk, nchunks); };
  auto tok_of = [&](const ChunkRef& cr) {
    return [=](int t) { return (cr.tok0 + (t < cr.tlen ? t : cr.tlen - 1)) * H + cr.h; };
  };
  auto load_in = [&](In& I, int64_t blk) {
    const ChunkRef cr = chunk_ref(blk);
    const auto tok = tok_of(cr);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t base = tok(4 * tg + r) * D + 8 * d8;
      I.kr[r] = gload_u4(kin, base);
      I.qr[r] = gload_u4(qin, base);
    }
    if (tid < C) {
      const int64_t ti = tok(tid);
      I.lds = ldin[ti];
      if (!FG2) I.gb = erin[ti];
    }
  };

  // The solve factor T stays in TH and is written out by the next chunk (or after the last),
  // so that the next chunk's wait for its inputs does not also wait for these stores.
  auto write_t = [&](int64_t pkt) { write_tri_t(ws + pkt * PK::bytes + PK::mat, TH, tid); };

  In I;
  int64_t blk = blockIdx.x;
  const int64_t gstride = gridDim.x;
  if (blk < nblk) load_in(I, blk);
  for (int64_t prev = -1; blk < nblk; blk += gstride) {
    const ChunkRef cr = chunk_ref(blk);
    char* pk = ws + cr.pkt * PK::bytes;  // this chunk's packet
    _Float16* wsc = reinterpret_cast<_Float16*>(pk + PK::mat);
    float* gv = reinterpret_cast<float*>(pk + PK::gate);
    // FG2: this thread's rates and values, issued with the chunk's other inputs
    float rt[FG2 ? 4 : 1][FG2 ? 8 : 1];
    uint4 vr[FG2 ? 4 : 1];
    if constexpr (FG2) {
      const gptr<const uint16_t> vin = opaque_gptr(static_cast<const uint16_t*>(p.v));
      const auto tok = tok_of(cr);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t base = tok(4 * tg + r) * D + 8 * d8;
        unpack8(gload_f4(erin, base), gload_f4(erin, base + 4), rt[r]);
        vr[r] = gload_u4(vin, base);
      }
    }
    vm_wait_all();  // this chunk's inputs (loaded one chunk ago) and the older stores

    uint4 kr[4], qr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = 4 * tg + r < cr.tlen;
      const uint4 z = make_uint4(0, 0, 0, 0);
      kr[r] = ok ? I.kr[r] : z;
      qr[r] = ok ? I.qr[r] : z;
    }
    float lds = 0.f;
    if (tid < C) {
      const bool ok = tid < cr.tlen;
      lds = ok ? I.lds : 0.f;
      GB[tid] = ok ? (FG2 ? 1.f : I.gb) : 0.f;
    }
    // chunk-local inclusive prefix sums of the log-decay (wave 0 lane t holds token t)
    if (wave == 0) {
      float x = lds;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      GSC[lane] = x;
    }
    // plain k and q (FG2: k~ = sqrt(beta) k), in LDS for the Gram products and in the packet for
    // the scan; FG2's v~ = sqrt(beta) v goes straight to the packet.  Rows past the end are zero.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * tg + r;
      float kf[8], qf[8];
      bf16x8_to_f32(kr[r], kf);
      bf16x8_to_f32(qr[r], qf);
      if constexpr (FG2) {
        const bool ok = t < cr.tlen;
        float vf[8];
        bf16x8_to_f32(vr[r], vf);
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          const float s = ok ? sqrtf(rt[r][ch]) : 0.f;
          kf[ch] *= s;
          vf[ch] *= s;
        }
        *reinterpret_cast<half8*>(pk + PK::vt + 2 * (t * D + 8 * d8)) = cvt8(vf);
      }
      const half8 hk = cvt8(kf), hq = cvt8(qf);
      *reinterpret_cast<half8*>(KP + t * KS + 8 * d8) = hk;
      *reinterpret_cast<half8*>(QP + t * KS + 8 * d8) = hq;
      *reinterpret_cast<half8*>(pk + PK::kp + 2 * swz<16>(t, 8 * d8)) = hk;
      *reinterpret_cast<half8*>(pk + PK::qp + 2 * swz<16>(t, 8 * d8)) = hq;
    }
    if (prev >= 0) write_t(prev);  // the previous chunk's T, still in TH
    lds_barrier();
    // gate vector: beta, and the scan's row factors relative to the chunk start (all <= 1)
    if (tid < C) {
      gv[GV_BETA + tid] = GB[tid];
      gv[GV_FP + tid] = __expf(GSC[tid]);
      gv[GV_FM + tid] = __expf(GSC[C - 1] - GSC[tid]);
    } else if (tid == C) {
      *reinterpret_cast<float4*>(gv + GV_SC) = make_float4(1.f, __expf(GSC[C - 1]), 1.f, 0.f);
    }
    for (int i = tid; i < C * CS; i += kThreads) TH[i] = (_Float16)0.f;

    // Gram tiles, transposed: lane gets A[t = 16 I + l16][i = 16 J + 4 lg + r].
    //   which 0: beta_t A_kk (strict), fp32 to LDS for the solve; 1: A_qk (lower), fp16 to the packet
    auto gram_tile = [&](int idx) {
      const int which = idx / 10;
      int I0, J0;
      tile_ij(idx - 10 * which, I0, J0);
      const _Float16* Bb = which == 1 ? QP : KP;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(frag(KP, KS, 16 * J0, 32 * ks, lane), frag(Bb, KS, 16 * I0, 32 * ks, lane), acc);
      const int t = 16 * I0 + l16;
      const int i0 = 16 * J0 + 4 * lg;
      // the decay between token i and token t >= i: e^{g_t - g_i} <= 1 (entries above the
      // diagonal are zeroed below)
      const float gt = GSC[t];
      const float4 gi = *reinterpret_cast<const float4*>(GSC + i0);
      acc[0] *= __expf(fminf(gt - gi.x, 0.f));
      acc[1] *= __expf(fminf(gt - gi.y, 0.f));
      acc[2] *= __expf(fminf(gt - gi.z, 0.f));
      acc[3] *= __expf(fminf(gt - gi.w, 0.f));
      if (which == 0) {
        const float sc = GB[t];
        float4 v;
        v.x = (i0 + 0 < t) ? sc * acc[0] : 0.f;
        v.y = (i0 + 1 < t) ? sc * acc[1] : 0.f;
        v.z = (i0 + 2 < t) ? sc * acc[2] : 0.f;
        v.w = (i0 + 3 < t) ? sc * acc[3] : 0.f;
        *reinterpret_cast<float4*>(AF + t * AFS + i0) = v;
        if (p.ck_A) {  // A_kk itself, for the gradients
          half4v hv;
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(i0 + r < t ? acc[r] : 0.f);
          *reinterpret_cast<half4v*>(static_cast<_Float16*>(p.ck_A) + cr.pkt * kAkkHalves + tri_pos(t, i0)) = hv;
        }
      } else {
        half4v hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(i0 + r <= t ? acc[r] : 0.f);
        *reinterpret_cast<half4v*>(wsc + PK::matb / 2 + tri_pos(t, i0)) = hv;
      }
    };
#pragma unroll
    for (int n = 0; n < 5; ++n) gram_tile(wave + 4 * n);
    // the upper-triangular 16 x 16 tiles (0,1) and (2,3) of A_qk share a stored block with
    // nonzeros and are zero (T's come from TH)
    if (wave < 2) {
      const half4v z = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
      const int I0 = 2 * wave, J0 = I0 + 1;
      *reinterpret_cast<half4v*>(wsc + PK::matb / 2 + tri_pos(16 * I0 + l16, 16 * J0 + 4 * lg)) = z;
      if (p.ck_A)
        *reinterpret_cast<half4v*>(static_cast<_Float16*>(p.ck_A) + cr.pkt * kAkkHalves +
                                   tri_pos(16 * I0 + l16, 16 * J0 + 4 * lg)) = z;
    }
    lds_barrier();
    // fetch the next chunk's inputs only now, in flight during the solve, which keeps them out of
    // the Gram stage's registers (measured faster)
    if (blk + gstride < nblk) load_in(I, blk + gstride);
    solve_t(AF, TH, tid);
    if (blk + gstride >= nblk) write_t(cr.pkt);  // this workgroup's last chunk
    prev = cr.pkt;
  }
}

// ------------------------------------------------------------------------------------------
// Prep with a per-channel decay or separate erase/write gates (KDA, Gated DeltaNet-2 /
// FG2-GDN+, FG2's rate with a per-channel decay).  Persistent like the scalar prep; two
// workgroups per compute unit.
//
// Every factor e^{x} that scales a matrix operand has x <= 0 (apart from the bounded midpoint
// split below), so fp16 operands stay in range for every decay in (0, 1]: a factor underflows
// only where the term it scales is itself negligible.
//  - The scan's tiles are referenced at the chunk start: K+ = k e^{g_t}, Q+ = q e^{g_t},
//    K^end = k e^{g_C - g_t} (and U^end for separate gates), with the state unscaled.
//  - The Gram matrices are built in 16-token blocks.  Block I's rows are referenced at the token
//    before the block, x_t e^{gl_t} (gl: the in-block inclusive prefix of the log-decay); the
//    columns of an earlier block J at the end of their own block, k_i e^{D_J - gl_i} (D_J: the
//    block's total), times the decay of the blocks strictly between them, e^{D_{J+1} + ...},
//    applied to the column fragment.
//  - A diagonal block is split at its log-midpoint, rows x_t e^{gl_t - D/2} and columns
//    k_i e^{D/2 - gl_i}, when its total decay is at most 12 on every channel (factors within
//    e^{+-6}) and its inputs are moderate; otherwise by levels: the pairs of the two halves of
//    16-, 8-, 4- and 2-token segments, each split at the boundary of its halves (factors <= 1),
//    plus the diagonal t = i with the plain operands.
//
// Lanes hold one token each: lane 16 lg + l16 of wave w holds token 16 w + l16 of the chunk and
// its channels 32 ks + 8 lg + j (ks, j = 0..3, 0..7), exactly the operand fragment layout of
// v_mfma_f32_16x16x32_f16, so the diagonal block of wave w is formed and multiplied in
// registers; the off-diagonal blocks read row and column operands written to LDS.
// ------------------------------------------------------------------------------------------
constexpr float kFastSpan = 12.f;  // largest per-channel log-decay of a block split at its midpoint
constexpr float kFastMag = 80.f;   // largest |k|, |q|, |u| there: 80 e^6 < 32768

// Inclusive prefix sum over the 16 lanes of each row (DPP row shifts; lanes without a source
// add zero).
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_prefix(float x) {
  x += dpp_row_shr<1>(x);
  x += dpp_row_shr<2>(x);
  x += dpp_row_shr<4>(x);
  x += dpp_row_shr<8>(x);
  return x;
}

// The value of lane (l & ~(S - 1)) | (S / 2 - 1) of each 16-lane row: the last token of the
// first half of this lane's S-token segment (ds_swizzle bit mode within 32 lanes).
template <int S>
__device__ __forceinline__ float seg_ref(float x) {
  constexpr int pattern = (0x10 | (0xf & ~(S - 1))) | ((S / 2 - 1) << 5);
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), pattern));
}

template <bool DCH, bool GEN, bool FG2>
__global__ __launch_bounds__(kThreads, 2) void chunk_prep_ch_kernel(Problem p, char* __restrict__ ws, int nchunks,
                                                                    int64_t nblk) {
  static_assert(DCH || GEN, "a per-head decay with one per-head gate runs chunk_prep_scalar_kernel");
  static_assert(!(FG2 && GEN), "the per-channel rate keeps the symmetric gates");
  if (p.chunks) nblk = int64_t(p.H) * *p.nchunks_total;
  using PK = Packet<DCH, GEN, FG2>;
  constexpr int NG = DCH ? 32 : 1;  // log-decays per lane
  // Gram products (row operand, column operand): 0 (k, k), 1 (q, k), 2 (k, u), 3 (q, u).  The
  // solve takes beta_t A_kk (symmetric gates) or A_ku; the packet holds A_qk (and A_kk, A_qu).
  constexpr int NP = GEN ? 4 : 2;
  constexpr int kSolveProd = GEN ? 2 : 0;

  __shared__ __attribute__((aligned(16))) _Float16 KR[C * D];          // row operands k e^{gl}
  __shared__ __attribute__((aligned(16))) float QRAF[C * AFS];         // row operands q e^{gl}, then AF
  __shared__ __attribute__((aligned(16))) _Float16 KC[48 * D];         // column operands k e^{D - gl}
  __shared__ __attribute__((aligned(16))) _Float16 UC[GEN ? 48 * D : 8];
  __shared__ __attribute__((aligned(16))) _Float16 TH[C * CS];
  __shared__ __attribute__((aligned(16))) float GSC[4 * D];            // block totals D_w
  __shared__ __attribute__((aligned(16))) float TW[4 * 3 * D];         // e^{g_b}, e^{g_C - g_e}, e^{-D/2}
  __shared__ __attribute__((aligned(16))) _Float16 FT[4 * D];          // e^{D_1}, e^{D_2}, e^{D_1 + D_2}, 1
  __shared__ float GB[C];
  static_assert(C * D * 2 <= C * AFS * 4, "the solve matrix takes the place of the q row operands");
  _Float16* const QR = reinterpret_cast<_Float16*>(QRAF);
  float* const AF = QRAF;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  const int tl = 16 * w + l16;  // this lane's token in the chunk
  const int H = p.H;
  const gptr<const uint16_t> kin = opaque_gptr(static_cast<const uint16_t*>(p.k));
  const gptr<const uint16_t> qin = opaque_gptr(static_cast<const uint16_t*>(p.q));
  const gptr<const uint16_t> vin = opaque_gptr(static_cast<const uint16_t*>(p.v));
  const gptr<const float> ldin = opaque_gptr(p.log_decay);
  const gptr<const float> erin = opaque_gptr(p.erase);
  const bool erase_ch = GEN && p.erase_channel;

  // One chunk's inputs for this lane's token (register c = 8 ks + j holds channel
  // 32 ks + 8 lg + j).  Tokens past the end load token T - 1 (zeroed where they are used), so
  // every load is unconditional.  No chunk is kept in flight: its registers would spill, and the
  // second resident workgroup covers the load latency (measured: prefetching the next chunk
  // during this chunk's Gram tiles and solve was 8-40% slower).
  constexpr bool ECH = GEN;  // erase gates held per channel (a per-head gate is repeated)
  struct In {
    uint4 kr[4], qr[4];
    float la[NG];
    float er[ECH ? 32 : 1];
    float bt;  // symmetric gates: the per-head erase/write gate
    float rt[FG2 ? 32 : 1];
    uint4 vr[FG2 ? 4 : 1];
  };
  auto load_in = [&](In& I, int64_t b) {
    const ChunkRef cr = chunk_ref_of(p, b, nchunks);
    const int64_t ti = (cr.tok0 + (tl < cr.tlen ? tl : cr.tlen - 1)) * H + cr.h;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int64_t base = ti * D + 32 * ks + 8 * lg;
      I.kr[ks] = gload_u4(kin, base);
      I.qr[ks] = gload_u4(qin, base);
      if constexpr (DCH) unpack8(gload_f4(ldin, base), gload_f4(ldin, base + 4), I.la + 8 * ks);
      if constexpr (FG2) {
        unpack8(gload_f4(erin, base), gload_f4(erin, base + 4), I.rt + 8 * ks);
        I.vr[ks] = gload_u4(vin, base);
      }
    }
    if constexpr (!DCH) I.la[0] = ldin[ti];
    if constexpr (GEN) {
      if (erase_ch) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int64_t base = ti * D + 32 * ks + 8 * lg;
          unpack8(gload_f4(erin, base), gload_f4(erin, base + 4), I.er + 8 * ks);
        }
      } else {
        const float e1 = erin[ti];
#pragma unroll
        for (int c = 0; c < 32; ++c) I.er[c] = e1;
      }
    }
    I.bt = (GEN || FG2) ? 1.f : erin[ti];
  };

  auto write_t = [&](int64_t pkt) { write_tri_t(ws + pkt * PK::bytes + PK::mat, TH, tid); };

  In I;
  for (int64_t blk = blockIdx.x, prev = -1; blk < nblk; blk += gridDim.x) {
    const ChunkRef cr = chunk_ref_of(p, blk, nchunks);
    char* pk = ws + cr.pkt * PK::bytes;
    _Float16* wsc = reinterpret_cast<_Float16*>(pk + PK::mat);
    float* gv = reinterpret_cast<float*>(pk + PK::gate);
    const bool ok = tl < cr.tlen;
    load_in(I, blk);

    // ---- this chunk's inputs, masked past the last token ---------------------------------
    // k and q stay packed (bf16; FG2: k~ as fp16) and are widened where they are used.  (Vectors
    // are selected component by component: a select of whole vectors becomes a select of their
    // addresses in scratch memory.)
    uint4 kr[4], qr[4];
    float gl[NG], ef[GEN ? 32 : 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kr[ks] = mask4(ok, I.kr[ks]);
      qr[ks] = mask4(ok, I.qr[ks]);
    }
#pragma unroll
    for (int c = 0; c < NG; ++c) gl[c] = ok ? I.la[c] : 0.f;
    if constexpr (GEN) {
#pragma unroll
      for (int c = 0; c < 32; ++c) ef[c] = ok ? I.er[c] : 0.f;
    }
    const float bt = ok ? I.bt : 0.f;
    // FG2: k~ = sqrt(beta) k replaces k (fp16 from here on); v~ = sqrt(beta) v goes straight to
    // the packet
    if constexpr (FG2) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float kf[8], vf[8];
        bf16x8_to_f32(kr[ks], kf);
        bf16x8_to_f32(I.vr[ks], vf);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float s = ok ? sqrtf(I.rt[8 * ks + j]) : 0.f;
          kf[j] *= s;
          vf[j] *= s;
        }
        kr[ks] = __builtin_bit_cast(uint4, cvt8(kf));
        *reinterpret_cast<half8*>(pk + PK::vt + 2 * (tl * D + 32 * ks + 8 * lg)) = cvt8(vf);
      }
    }
    // channels 32 ks + 8 lg + 0..7 of k and q, widened
    auto kval = [&](int ks, float* f) {
      if constexpr (FG2) {
        const half8 h = __builtin_bit_cast(half8, kr[ks]);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = float(h[j]);
      } else {
        bf16x8_to_f32(kr[ks], f);
      }
    };
    auto qval = [&](int ks, float* f) { bf16x8_to_f32(qr[ks], f); };
    // eight floats of an LDS table at channel 32 ks + 8 lg
    auto lds8 = [&](const float* base, int ks, float* f) {
      unpack8(*reinterpret_cast<const float4*>(base + 32 * ks + 8 * lg),
              *reinterpret_cast<const float4*>(base + 32 * ks + 8 * lg + 4), f);
    };

    // ---- in-block prefix sums, block totals --------------------------------------------
#pragma unroll
    for (int c = 0; c < NG; ++c) gl[c] = row_prefix(gl[c]);
    if (l16 == 15) {
      if constexpr (DCH) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          *reinterpret_cast<float4*>(GSC + w * D + 32 * ks + 8 * lg) =
              make_float4(gl[8 * ks], gl[8 * ks + 1], gl[8 * ks + 2], gl[8 * ks + 3]);
          *reinterpret_cast<float4*>(GSC + w * D + 32 * ks + 8 * lg + 4) =
              make_float4(gl[8 * ks + 4], gl[8 * ks + 5], gl[8 * ks + 6], gl[8 * ks + 7]);
        }
      } else if (lg == 0) {
        GSC[w * D] = gl[0];
      }
    }
    if (lg == 0) GB[tl] = bt;
    if (prev >= 0) write_t(prev);  // the previous chunk's T, still in TH
    lds_barrier();

    // ---- per-block factors, gate vector ------------------------------------------------
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = lane + 64 * i, dd = DCH ? d : 0;
      const float D0 = GSC[dd], D1 = GSC[D + dd], D2 = GSC[2 * D + dd], D3 = GSC[3 * D + dd];
      const float Dw = w == 0 ? D0 : w == 1 ? D1 : w == 2 ? D2 : D3;
      const float after = (w < 1 ? D1 : 0.f) + (w < 2 ? D2 : 0.f) + (w < 3 ? D3 : 0.f);
      const float before = (w > 0 ? D0 : 0.f) + (w > 1 ? D1 : 0.f) + (w > 2 ? D2 : 0.f);
      TW[(3 * w + 0) * D + d] = __expf(before);
      TW[(3 * w + 1) * D + d] = __expf(after);
      TW[(3 * w + 2) * D + d] = __expf(-0.5f * Dw);
      if (w == 0) {
        FT[d] = (_Float16)__expf(D1);
        FT[D + d] = (_Float16)__expf(D2);
        FT[2 * D + d] = (_Float16)__expf(D1 + D2);
        FT[3 * D + d] = (_Float16)1.f;
      } else if (w == 1) {
        gv[GV_EM + d] = 1.f;
        gv[GV_FC + d] = __expf(D0 + D1 + D2 + D3);
        gv[GV_FCM + d] = 1.f;
      } else if (w == 2 && i == 0) {
        int ln = lane;  // (through an empty asm: the address is formed here, not kept in a register)
        asm volatile("" : "+v"(ln));
        gv[GV_BETA + ln] = GB[ln];
      }
    }
    for (int i = tid; i < C * CS; i += kThreads) TH[i] = (_Float16)0.f;
    // (the wave reads back only table rows its own lanes wrote above)
    const float* Dwt = GSC + w * D;            // this wave's block total per channel
    const float* TB = TW + 3 * w * D;          // e^{g before the block}
    const float* TA = TW + (3 * w + 1) * D;    // e^{g_C - g at the block's end}
    const float* TM = TW + (3 * w + 2) * D;    // e^{-D/2}

    // ---- operand tiles and the diagonal block, 32 channels at a time -----------------------
    // The diagonal block's contraction over channels splits into independent 32-channel slices,
    // so each slice takes the midpoint split when its block decay is at most kFastSpan on every
    // channel and its inputs are moderate, and the level split otherwise (NaN takes the level
    // split, and propagates).  Lane (lg, l16) accumulates the block's A[t = l16][i = 4 lg + r]
    // (block-local) of each product.
    f32x4 dacc[NP];
#pragma unroll
    for (int n = 0; n < NP; ++n) dacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float kf[8], qf[8], uf[8], dw[8], tb[8], ta[8], tm[8];
      kval(ks, kf);
      qval(ks, qf);
      if constexpr (DCH) {
        lds8(Dwt, ks, dw);
        lds8(TB, ks, tb);
        lds8(TA, ks, ta);
        lds8(TM, ks, tm);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          dw[j] = Dwt[0];
          tb[j] = TB[0];
          ta[j] = TA[0];
          tm[j] = TM[0];
        }
      }
      bool bad = false;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uf[j] = GEN ? ef[GEN ? 8 * ks + j : 0] * kf[j] : 0.f;
        bad |= !(dw[j] >= -kFastSpan);
        bad |= !(fabsf(kf[j]) <= kFastMag) || !(fabsf(qf[j]) <= kFastMag);
        if constexpr (GEN) bad |= !(fabsf(uf[j]) <= kFastMag);
      }
      const bool fast = __ballot(bad) == 0;
      float eg[8], edg[8];  // e^{gl} and e^{D - gl}, both <= 1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float g = gl[DCH ? 8 * ks + j : 0];
        eg[j] = __expf(g);
        edg[j] = __expf(dw[j] - g);
      }
      // each tile formed, converted and stored in turn (kept apart, the eight would not fit in
      // registers): scan tiles k e^{g_t}, q e^{g_t}, k e^{g_C - g_t} (, u e^{g_C - g_t}) to the
      // packet; Gram operands k e^{gl}, q e^{gl}, k e^{D - gl} (, u e^{D - gl}) to LDS
      auto put = [&](auto&& f, void* dst) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = f(j);
        *reinterpret_cast<half8*>(dst) = cvt8(x);
      };
      const int po = 2 * swz<16>(tl, 32 * ks + 8 * lg);  // byte offset in a packet tile
      const int lo = swz<16>(tl, 32 * ks + 8 * lg);      // half offset in an LDS tile
      put([&](int j) { return kf[j] * (eg[j] * tb[j]); }, pk + PK::kp + po);
      put([&](int j) { return qf[j] * (eg[j] * tb[j]); }, pk + PK::qp + po);
      put([&](int j) { return kf[j] * (edg[j] * ta[j]); }, pk + PK::kmt + po);
      if constexpr (GEN) put([&](int j) { return uf[j] * (edg[j] * ta[j]); }, pk + PK::umt + po);
      put([&](int j) { return kf[j] * eg[j]; }, KR + lo);
      put([&](int j) { return qf[j] * eg[j]; }, QR + lo);
      if (w < 3) {
        put([&](int j) { return kf[j] * edg[j]; }, KC + lo);
        if constexpr (GEN) put([&](int j) { return uf[j] * edg[j]; }, UC + lo);
      }
      // lane: A[row = i (this token)][k = 8 lg + j] and B[k][col = t (this token)]
      auto products = [&](const half8& rk, const half8& rq, const half8& ck, const half8& cu, f32x4 (&acc)[NP]) {
        acc[0] = mfma16x16x32(ck, rk, acc[0]);
        acc[1] = mfma16x16x32(ck, rq, acc[1]);
        if constexpr (GEN) {
          acc[2] = mfma16x16x32(cu, rk, acc[2]);
          acc[3] = mfma16x16x32(cu, rq, acc[3]);
        }
      };
      if (fast) {
        float rk8[8], rq8[8], ck8[8], cu8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float er = eg[j] * tm[j], ec = edg[j] * tm[j];  // e^{gl - D/2}, e^{D/2 - gl}
          rk8[j] = kf[j] * er;
          rq8[j] = qf[j] * er;
          ck8[j] = kf[j] * ec;
          cu8[j] = uf[j] * ec;
        }
        products(cvt8(rk8), cvt8(rq8), cvt8(ck8), cvt8(cu8), dacc);
      } else {
        // levels: segments of S tokens, rows in the second half, columns in the first, both
        // referenced at the last token of the first half (factors <= 1); the pairs of other
        // segments that also meet in a product are masked out
        auto level = [&](auto seg) {
          constexpr int S = decltype(seg)::value;
          const bool is_row = (l16 & (S - 1)) >= S / 2;
          float rk8[8], rq8[8], ck8[8], cu8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float g = gl[DCH ? 8 * ks + j : 0];
            const float gr = seg_ref<S>(g);
            const float f = __expf(is_row ? g - gr : gr - g);
            rk8[j] = is_row ? kf[j] * f : 0.f;
            rq8[j] = is_row ? qf[j] * f : 0.f;
            ck8[j] = is_row ? 0.f : kf[j] * f;
            cu8[j] = is_row ? 0.f : uf[j] * f;
          }
          f32x4 lacc[NP];
#pragma unroll
          for (int n = 0; n < NP; ++n) lacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
          products(cvt8(rk8), cvt8(rq8), cvt8(ck8), cvt8(cu8), lacc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool same = (l16 / S) == ((4 * lg + r) / S);
#pragma unroll
            for (int n = 0; n < NP; ++n) dacc[n][r] += same ? lacc[n][r] : 0.f;
          }
        };
        level(IntTag<16>());
        level(IntTag<8>());
        level(IntTag<4>());
        level(IntTag<2>());
        // the diagonal t = i with the plain operands
        f32x4 lacc[NP];
#pragma unroll
        for (int n = 0; n < NP; ++n) lacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        const half8 hk = cvt8(kf);
        products(hk, cvt8(qf), hk, cvt8(uf), lacc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int n = 0; n < NP; ++n) dacc[n][r] += (l16 == 4 * lg + r) ? lacc[n][r] : 0.f;
      }
    }
    lds_barrier();  // row and column operands, FT, TH cleared

    // ---- Gram tiles ----------------------------------------------------------------------
    // Off-diagonal tile n = 0..5: (I, J) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2), transposed:
    // lane gets A[t = 16 I + l16][i = 16 J + 4 lg + r].  The column fragments of the tiles two or
    // three blocks apart are scaled by the decay of the blocks between (FT rows 0..2; row 3 is one).
    auto off_tile = [&](int n, int prod) {
      const int I = n < 1 ? 1 : n < 3 ? 2 : 3;
      const int J = n - (I * (I - 1)) / 2;
      const _Float16* rowb = (prod & 1) ? QR : KR;
      const _Float16* colb = (prod & 2) ? UC : KC;
      const int fi = n == 1 ? 0 : n == 4 ? 1 : n == 3 ? 2 : 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const half8 a = frag_s<16>(colb, 16 * J, 32 * ks, lane) *
                        *reinterpret_cast<const half8*>(FT + fi * D + 32 * ks + 8 * lg);
        acc = mfma16x16x32(a, frag_s<16>(rowb, 16 * I, 32 * ks, lane), acc);
      }
      return acc;
    };
    // packet matrix of product n (1: A_qk, 2: A_kk, 3: A_qu); strict: A_kk
    auto pkt_mat = [&](int prod) { return prod == 1 ? 1 : prod == 0 ? 2 : 3; };
    auto store_pkt = [&](int prod, int t, int i0, f32x4 acc, bool diag) {
      const bool strict = prod == 0;
      half4v hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (_Float16)((!diag || (strict ? i0 + r < t : i0 + r <= t)) ? acc[r] : 0.f);
      *reinterpret_cast<half4v*>(wsc + pkt_mat(prod) * (PK::matb / 2) + tri_pos(t, i0)) = hv;
    };
    auto store_af = [&](int t, int i0, f32x4 acc, bool diag) {
      const float sc = GEN ? 1.f : GB[t];
      float4 v;
      v.x = (!diag || i0 + 0 < t) ? sc * acc[0] : 0.f;
      v.y = (!diag || i0 + 1 < t) ? sc * acc[1] : 0.f;
      v.z = (!diag || i0 + 2 < t) ? sc * acc[2] : 0.f;
      v.w = (!diag || i0 + 3 < t) ? sc * acc[3] : 0.f;
      *reinterpret_cast<float4*>(AF + t * AFS + i0) = v;
    };
    // phase A: the packet's products (they read the q row operands, which the solve matrix
    // overwrites in phase B)
    {
      constexpr int NA = GEN ? 18 : 6;  // (tile, product) pairs
      // (rolled: unrolled, the fragment reads of all of a wave's tiles are hoisted together and
      // spill)
#pragma unroll 1
      for (int m = 0; m < (NA + 3) / 4; ++m) {
        const int x = w + 4 * m;
        if (x < NA) {
          const int n = x % 6, a = x / 6;
          const int prod = GEN ? (a == 0 ? 0 : a == 1 ? 1 : 3) : 1;
          const int I = n < 1 ? 1 : n < 3 ? 2 : 3;
          const int J = n - (I * (I - 1)) / 2;
          store_pkt(prod, 16 * I + l16, 16 * J + 4 * lg, off_tile(n, prod), false);
        }
      }
      const int t = tl, i0 = 16 * w + 4 * lg;
      store_pkt(1, t, i0, dacc[1], true);
      if constexpr (GEN) {
        store_pkt(0, t, i0, dacc[0], true);
        store_pkt(3, t, i0, dacc[3], true);
      }
      // the upper-triangular 16 x 16 tiles (0,1) and (2,3) of the packet matrices after T share
      // a stored block with nonzeros and are zero
      for (int n = w; n < 2 * (PK::nmat - 1); n += 4) {
        const half4v z = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
        const int m = 1 + n / 2, I0 = 2 * (n % 2), J0 = I0 + 1;
        *reinterpret_cast<half4v*>(wsc + m * (PK::matb / 2) + tri_pos(16 * I0 + l16, 16 * J0 + 4 * lg)) = z;
      }
    }
    lds_barrier();
    // phase B: the solve matrix, fp32, over the q row operands (one per-head gate: A_kk also to
    // the gradients' side buffer when it is given)
    _Float16* const cka = (!GEN && p.ck_A) ? static_cast<_Float16*>(p.ck_A) + cr.pkt * kAkkHalves : nullptr;
    auto store_cka = [&](int t, int i0, f32x4 acc, bool diag) {
      half4v hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (_Float16)((!diag || i0 + r < t) ? acc[r] : 0.f);
      *reinterpret_cast<half4v*>(cka + tri_pos(t, i0)) = hv;
    };
    for (int n = w; n < 6; n += 4) {
      const int I = n < 1 ? 1 : n < 3 ? 2 : 3;
      const int J = n - (I * (I - 1)) / 2;
      const f32x4 a = off_tile(n, kSolveProd);
      store_af(16 * I + l16, 16 * J + 4 * lg, a, false);
      if (cka) store_cka(16 * I + l16, 16 * J + 4 * lg, a, false);
    }
    store_af(tl, 16 * w + 4 * lg, dacc[kSolveProd], true);
    if (cka) {
      store_cka(tl, 16 * w + 4 * lg, dacc[kSolveProd], true);
      if (w < 2) {
        const half4v z = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
        *reinterpret_cast<half4v*>(cka + tri_pos(32 * w + l16, 32 * w + 16 + 4 * lg)) = z;
      }
    }
    lds_barrier();
    solve_t(AF, TH, tid);
    if (blk + gridDim.x >= nblk) write_t(cr.pkt);  // this workgroup's last chunk
    prev = cr.pkt;
  }
}

// ------------------------------------------------------------------------------------------
// Scan: the chunks of one (b, h, value slice) in order, eight waves per workgroup.
// ------------------------------------------------------------------------------------------
constexpr int kScanWaves = 8;
constexpr int kScanThreads = 64 * kScanWaves;

// LDS layout of the register-staged scan (general gates).
template <bool GEN, bool SCAL, int DVS>
struct ScanLayout {
  static_assert(GEN && !SCAL, "the register-staged scan serves general gates");
  // Every tile in the packet's layout (swizzled, see swz_key; the matrices as 16 x 32 blocks, see
  // tri_pos), so units copy straight across and fragment reads are conflict-free.
  static constexpr int kp = 0;                 // K+       [64][128] half
  static constexpr int qp = kp + C * D * 2;    // Q+       [64][128]
  static constexpr int kmt = qp + C * D * 2;   // K^end    [64][128]
  static constexpr int umt = kmt + D * C * 2;  // U^end    [64][128]
  static constexpr int st = umt + D * C * 2;   // S~^T     [DVS][128]
  // the four lower-triangular matrices: eight 16 x 32 blocks each (see tri_pos), contiguous
  static constexpr int th = st + DVS * D * 2;  // T        [64][64]
  static constexpr int aq = th + C * C * 2;    // A_qk     [64][64]
  static constexpr int akk = aq + C * C * 2;   // A_kk     [64][64]
  static constexpr int aqu = akk + C * C * 2;  // A_qu     [64][64]
  static constexpr int rt = aqu + C * C * 2;   // Y^T      [DVS][64]
  static constexpr int dt = rt + DVS * C * 2;  // (-M)^T   [DVS][64]
  static constexpr int vt = dt + DVS * C * 2;  // Vt^T     [DVS][64]
  static constexpr int total = vt + DVS * C * 2;
};

// Value-slice words per thread: DVS/8 bf16 values.
template <int DVS> struct VSlice;
template <> struct VSlice<16> { uint32_t w; };
template <> struct VSlice<32> { uint2 w; };
template <> struct VSlice<64> { uint4 w; };

template <int DVS>
__device__ __forceinline__ void vslice_load(VSlice<DVS>& v, gptr<const uint16_t> base, int64_t i, bool ok) {
  if constexpr (DVS == 16) {
    v.w = ok ? *(gptr<const uint32_t>)(base + i) : 0u;
  } else if constexpr (DVS == 32) {
    v.w = ok ? gload_u2(base, i) : make_uint2(0, 0);
  } else {
    v.w = ok ? gload_u4(base, i) : make_uint4(0, 0, 0, 0);
  }
}

template <int DVS>
__device__ __forceinline__ void vslice_f32(const VSlice<DVS>& v, float* f) {
  if constexpr (DVS == 16) {
    f[0] = __uint_as_float(v.w << 16); f[1] = __uint_as_float(v.w & 0xffff0000u);
  } else if constexpr (DVS == 32) {
    f[0] = __uint_as_float(v.w.x << 16); f[1] = __uint_as_float(v.w.x & 0xffff0000u);
    f[2] = __uint_as_float(v.w.y << 16); f[3] = __uint_as_float(v.w.y & 0xffff0000u);
  } else {
    bf16x8_to_f32(v.w, f);
  }
}

// Compile-time flag passed to generic lambdas.
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Scan, general gates (separate erase and write gates): the packet (too large for two LDS
// buffer sets) is staged through registers one or two chunks ahead.  WCH: per-channel write
// gate.
// CKPT: also store the state at the start of every chunk (p.ck_S, for the gradients).
template <bool DCH, bool GEN, bool WCH, int DVS, bool CKPT = false>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(Problem p, const char* __restrict__ ws) {
  static_assert(GEN, "symmetric gates use chunk_scan_sym_kernel");
  using PK = Packet<DCH, GEN>;
  using L = ScanLayout<GEN, false, DVS>;
  constexpr int NM = PK::nmat;
  constexpr int NCT = DVS / 16;   // 16-column tiles of the value slice
  constexpr int VPT = DVS / 8;    // value columns per thread in the V load
  constexpr int NTU = 8;  // 16-byte operand-tile units per thread (K+, Q+, K^end, U^end)
  constexpr int PF = 2;   // chunks of prefetch in flight (one register set each)
  __shared__ __attribute__((aligned(16))) char smem[L::total];
  _Float16* KP = reinterpret_cast<_Float16*>(smem + L::kp);
  _Float16* QP = reinterpret_cast<_Float16*>(smem + L::qp);
  _Float16* KMT = reinterpret_cast<_Float16*>(smem + L::kmt);
  _Float16* UMT = reinterpret_cast<_Float16*>(smem + L::umt);
  _Float16* ST = reinterpret_cast<_Float16*>(smem + L::st);
  _Float16* TH = reinterpret_cast<_Float16*>(smem + L::th);
  _Float16* AQ = reinterpret_cast<_Float16*>(smem + L::aq);
  _Float16* AKK = reinterpret_cast<_Float16*>(smem + L::akk);
  _Float16* AQU = reinterpret_cast<_Float16*>(smem + L::aqu);
  _Float16* RT = reinterpret_cast<_Float16*>(smem + L::rt);
  _Float16* DT = reinterpret_cast<_Float16*>(smem + L::dt);
  _Float16* VT = reinterpret_cast<_Float16*>(smem + L::vt);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int H = p.H;
  const WgRef wg = wg_ref(p);
  const int bh = wg.bh, h = bh % H;
  const int j0 = wg.slice * DVS;
  const SeqRef sq = seq_ref(p, bh, h);
  const int T = sq.len;  // this sequence's tokens
  const int nchunks = sq.nch;
  if (nchunks == 0) {
    pass_state(p, bh, j0, DVS);
    return;
  }
  const int nfull = T / C;  // chunks with C tokens
  const gptr<const uint16_t> vin = opaque_gptr(static_cast<const uint16_t*>(p.v));
  const gptr<const float> wrin = opaque_gptr(p.write);
  const gptr<const char> pbase = opaque_gptr(ws) + sq.pkt0 * PK::bytes;

  // State: wave w owns rows [16 w, 16 w + 16) x the DVS columns as NCT accumulator tiles
  // (lane: column 16 ct + l16, rows 16 w + 4 lg + r).
  f32x4 S[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = 16 * wave + 4 * lg + r;
      S[ct][r] = p.S0 ? p.S0[(int64_t(bh) * D + d) * D + j0 + 16 * ct + l16] : 0.f;
    }

  // Load mapping.  Packet tiles: 16-byte units tid and tid + 512; matrices: unit tid.  Value
  // slice: token tid / 8, columns VPT (tid % 8) .. + VPT - 1.
  const int vtok = tid >> 3, vcol = (tid & 7) * VPT;
  auto tok = [&](int t) { return (sq.tok0 + t) * H + h; };
  // Per-thread element offsets at chunk 0; chunk c adds c * tstride (tokens are H * D apart).
  const int64_t tstride = int64_t(C) * H * D;
  const int64_t v_off = tok(vtok) * D + j0 + vcol;
  const int64_t w_off = tok(vtok);
  const int64_t o_off = tok(16 * (wave & 3) + l16) * D + j0 + 4 * lg;
  // Tokens past the end load token T - 1 instead (the values are zeroed where they are used), so
  // that every load is issued unconditionally and the wait counts stay exact.
  const int64_t v_last = tok(T - 1) * D + j0 + vcol;
  const int64_t w_last = tok(T - 1);

  struct Pref {
    uint4 mr[NM * 3 / 4];     // this thread's units of the stored blocks of T, A_qk, A_kk, A_qu
    uint4 tl[NTU];            // K+, Q+, K^end, U^end units
    float4 sc[3];             // per-channel state factors (1, e^{g_C}, 1) of this thread's 4 rows
    VSlice<DVS> vr;
    float wr[GEN ? VPT : 1];  // write gates of the value slice (per channel) or of token vtok
  };

  // The loads of one chunk are issued in three batches, one per compute stage, so that the
  // vector-memory path stays busy without stalling every wave at one point.
  auto load_a = [&](Pref& P, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      P.tl[i] = ldb16(pk, PK::kp + 16 * (tid + kScanThreads * i));
      P.tl[2 + i] = ldb16(pk, PK::qp + 16 * (tid + kScanThreads * i));
    }
    const int d0 = 16 * wave + 4 * lg;
    P.sc[0] = ldf16(pk, PK::gate + 4 * (GV_EM + d0));
    P.sc[1] = ldf16(pk, PK::gate + 4 * (GV_FC + d0));
    P.sc[2] = ldf16(pk, PK::gate + 4 * (GV_FCM + d0));
  };
  auto load_b = [&](Pref& P, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
#pragma unroll
    for (int j = 0; j < NM * 3 / 4; ++j) P.mr[j] = ldb16(pk, PK::mat + 16 * (tid + kScanThreads * j));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      P.tl[4 + i] = ldb16(pk, PK::kmt + 16 * (tid + kScanThreads * i));
      P.tl[6 + i] = ldb16(pk, PK::umt + 16 * (tid + kScanThreads * i));
    }
  };
  auto load_c = [&](Pref& P, int c) {
    const bool ok = c * C + vtok < T;
    const int64_t vb = ok ? v_off + c * tstride : v_last;
    vslice_load<DVS>(P.vr, vin, vb, true);
    if constexpr (GEN) {
      if constexpr (WCH) {
        if constexpr (VPT == 2) {
          const f32x2 w2 = *(gptr<const f32x2>)(wrin + vb);
          P.wr[0] = w2.x;
          P.wr[1] = w2.y;
        } else {
#pragma unroll
          for (int i = 0; i < VPT; i += 4) {
            const float4 w4 = gload_f4(wrin, vb + i);
            P.wr[i] = w4.x; P.wr[i + 1] = w4.y; P.wr[i + 2] = w4.z; P.wr[i + 3] = w4.w;
          }
        }
      } else {
        P.wr[0] = wrin[ok ? w_off + int64_t(c) * C * H : w_last];
      }
    }
  };

  // TAIL: the chunk may extend past the last token (its output rows are masked).  Full chunks
  // store unconditionally, so that the stores do not make the wait counts of later loads
  // conservative.
  auto step = [&](auto tail, int c, Pref& P) {
    constexpr bool TAIL = decltype(tail)::value;
    if constexpr (CKPT) store_state_h(static_cast<_Float16*>(p.ck_S) + (sq.pkt0 + c) * D * D, j0, S);
    // ---- L: the chunk's packet, value slice and S~^T into LDS ------------------------------
    // the LDS tiles keep the packet's layout: 16-byte units copy straight across
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kScanThreads * i;
      *reinterpret_cast<uint4*>(KP + 8 * u) = P.tl[i];
      *reinterpret_cast<uint4*>(QP + 8 * u) = P.tl[2 + i];
      *reinterpret_cast<uint4*>(KMT + 8 * u) = P.tl[4 + i];
      *reinterpret_cast<uint4*>(UMT + 8 * u) = P.tl[6 + i];
    }
    // stored block k of matrix m (1 KB each, see tri_pos) to LDS block 2 I + H of that matrix
#pragma unroll
    for (int j = 0; j < NM * 3 / 4; ++j) {
      const int u = tid + kScanThreads * j, m = u / 384, k = (u % 384) / 64;
      const int lb = k < 2 ? 2 * k : k + 2;
      *reinterpret_cast<uint4*>(TH + 4096 * m + 512 * lb + 8 * (u % 64)) = P.mr[j];
    }
    {
      float vf[VPT];
      vslice_f32<DVS>(P.vr, vf);
      const bool vok = c * C + vtok < T;
#pragma unroll
      for (int i = 0; i < VPT; ++i) vf[i] = vok ? vf[i] : 0.f;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const float w = WCH ? P.wr[i] : P.wr[0];
        VT[swz<8>(vcol + i, vtok)] = (_Float16)(w * vf[i]);
      }
    }
    // S~^T = (Diag(em) S)^T (em = 1: the tiles are referenced at the chunk start); the end-of-chunk
    // factors of this wave's rows stay in registers.
    float fC[4], fCm[4];
    {
      float em[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        em[r] = (&P.sc[0].x)[r];
        fC[r] = (&P.sc[1].x)[r];
        fCm[r] = (&P.sc[2].x)[r];
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        half4v hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(em[r] * S[ct][r]);
        *reinterpret_cast<half4v*>(ST + swz<16>(16 * ct + l16, 16 * wave + 4 * lg)) = hv;
      }
    }
    lds_barrier();
    // next chunks' loads (past the last chunk: reload the last one, unused)
    const int cn = c + PF < nchunks ? c + PF : nchunks - 1;
    load_a(P, cn);

    // ---- X = [K+; Q+] S~ ----------------------------------------------------------------
    // waves 0-3: X_K rows [16 w, +16); waves 4-7: X_Q rows [16 (w - 4), +16), transposed.
    const int xrow = 16 * (wave & 3);
    const bool xq_wave = wave >= 4;
    f32x4 XR[NCT];
    {
      const _Float16* Xa = xq_wave ? QP : KP;
      half8 af[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) af[ks] = frag_s<16>(Xa, xrow, 32 * ks, lane);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // X_K as is (lane: rows t, column j); X_Q transposed (lane: rows j, column t) so that
        // the output tile it seeds can be stored as 16-byte rows of o.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const half8 bs = frag_s<16>(ST, 16 * ct, 32 * ks, lane);
          // the wave-dependent operand order is a choice of operands for one product: two
          // products behind a branch gave wrong results in one register allocation
          const half8 opa = xq_wave ? bs : af[ks], opb = xq_wave ? af[ks] : bs;
          acc = mfma16x16x32(opa, opb, acc);
        }
        XR[ct] = acc;
      }
    }
    // (no barrier: the X stage writes no LDS, and Y reads only tiles stored before the last one)

    // Y = X_K + A_kk Vt, stored transposed (B operand of M = T Y); A_kk has zero upper tiles,
    // so both halves of the product run unconditionally
    if (!xq_wave) {
      half8 ka[2], vb[NCT][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ka[ks] = frag_tri(AKK, xrow / 16, ks, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) vb[ct][ks] = frag_s<8>(VT, 16 * ct, 32 * ks, lane);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 y = XR[ct];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) y = mfma16x16x32(ka[ks], vb[ct][ks], y);
        half4v hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (_Float16)y[r];
        *reinterpret_cast<half4v*>(RT + swz<8>(16 * ct + l16, xrow + 4 * lg)) = hv;
      }
    }
    lds_barrier();

    load_b(P, cn);
    // ---- D: delta = T R (symmetric) or -M = -(T Y) (general), stored transposed ---------
#pragma unroll
    for (int n = wave; n < 4 * NCT; n += kScanWaves) {
      const int i = n & 3, ct = n >> 2;
      // T has zero upper tiles: both halves, no branch
      half8 ta[2], yb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ta[ks] = frag_tri(TH, i, ks, lane);
        yb[ks] = frag_s<8>(RT, 16 * ct, 32 * ks, lane);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma16x16x32(ta[ks], yb[ks], acc);
      half4v hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(-acc[r]);
      *reinterpret_cast<half4v*>(DT + swz<8>(16 * ct + l16, 16 * i + 4 * lg)) = hv;
      if constexpr (CKPT) {
        if (p.ck_M) store_rows(p.ck_M, sq.pkt0 + c, 16 * i + 4 * lg, j0 + 16 * ct + l16, acc);
      }
    }
    lds_barrier();

    load_c(P, cn);
    // ---- O: chunk output rows [16 (w - 4), +16), waves 4-7 --------------------------------
    if (xq_wave) {
      // O^T tile: lane holds O[t = 16 i + l16][j = 16 ct + 4 lg + 0..3]
      const int i = wave & 3;
      const int t = c * C + 16 * i + l16;
      // A_qk and A_qu have zero upper tiles: both halves, no branch
      half8 bq[2], bu[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bq[ks] = frag_tri(AQ, i, ks, lane);
        bu[ks] = frag_tri(AQU, i, ks, lane);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = XR[ct];
        half8 va[2], da[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          va[ks] = frag_s<8>(VT, 16 * ct, 32 * ks, lane);
          da[ks] = frag_s<8>(DT, 16 * ct, 32 * ks, lane);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          acc = mfma16x16x32(va[ks], bq[ks], acc);
          acc = mfma16x16x32(da[ks], bu[ks], acc);
        }
        if (!TAIL || t < T) store_o4(p.o, o_off + c * tstride + 16 * ct, acc, p.o_bf16);
      }
    }

    // ---- S: state update for this wave's rows ---------------------------------------------
    {
      f32x4 acc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      half8 ak[2], au[2], bv[NCT][2], bd[NCT][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ak[ks] = frag_ts(KMT, 16 * wave, 32 * ks, lane);
        au[ks] = frag_ts(UMT, 16 * wave, 32 * ks, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          bv[ct][ks] = frag_s<8>(VT, 16 * ct, 32 * ks, lane);
          bd[ct][ks] = frag_s<8>(DT, 16 * ct, 32 * ks, lane);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          acc[ct] = mfma16x16x32(ak[ks], bv[ct][ks], acc[ct]);
          acc[ct] = mfma16x16x32(au[ks], bd[ct][ks], acc[ct]);
        }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[ct][r] = fmaf(fC[r], S[ct][r], fCm[r] * acc[ct][r]);
    }
    lds_barrier();
  };

  auto load = [&](Pref& P, int c) {
    load_a(P, c);
    load_b(P, c);
    load_c(P, c);
  };
  // the upper blocks (0,1) and (1,1) of the four matrices are zero and never copied
  *reinterpret_cast<uint4*>(TH + 4096 * (tid >> 7) + 512 * (1 + 2 * ((tid >> 6) & 1)) + 8 * lane) =
      make_uint4(0, 0, 0, 0);
  // chunk c's inputs sit in set c % 2; each step refills its set with chunk c + 2
  Pref PA, PB;
  load(PA, 0);
  load(PB, nchunks > 1 ? 1 : 0);
  int c = 0;
  for (; c + 1 < nfull; c += 2) {
    step(Flag<false>(), c, PA);
    step(Flag<false>(), c + 1, PB);
  }
  if (c < nfull) step(Flag<false>(), c++, PA);
  if (c < nchunks) {
    if (c & 1) step(Flag<true>(), c, PB);
    else step(Flag<true>(), c, PA);
  }

  if (p.S_T) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * wave + 4 * lg + r;
        p.S_T[(int64_t(bh) * D + d) * D + j0 + 16 * ct + l16] = S[ct][r];
      }
  }
}


// ------------------------------------------------------------------------------------------
// Scan, symmetric gates (one per-head erase/write gate): the chunks of one (b, h, value slice)
// in order, eight waves per workgroup.  The packet tiles of chunk c + 1 are copied global ->
// LDS by the load-to-LDS path (no registers, no VALU) into the second of two buffer sets while
// chunk c is computed from the first; each chunk starts with one wait for its own copies.
// ------------------------------------------------------------------------------------------
// FG2: the values are FG2's v~ = sqrt(beta) v, fp16 in the packet, instead of the bf16 input.
template <bool DCH, int DVS, bool FG2 = false, bool CKPT = false>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_sym_kernel(Problem p, const char* __restrict__ ws) {
  using PK = Packet<DCH, false, FG2>;
  auto vval = [](uint16_t u) { return FG2 ? float(__builtin_bit_cast(_Float16, u)) : bf16_to_f32(u); };
  constexpr bool SCAL = !DCH;
  constexpr int NCT = DVS / 16;  // 16-column tiles of the value slice
  constexpr int VU = DVS / 8;    // 16-byte units per value-slice row
  // Two buffer sets of copy targets, each split into one array per copy batch: the compiler
  // tracks copies into LDS per array, so reading one array never waits for the copies into
  // another.  Batch 1a (bytes): K+ (scalar decay: k) [64][128]; batch 1b: Q+ (q) [64][128],
  // gate vector [ngate] f32, v slice [64][DVS] (bf16); batch 2: T [64][64], A_qk [64][64]
  // (eight 16 x 32 blocks each, see tri_pos); batch 3: K^end [64][128] (per-channel decay).
  constexpr int b1a_bytes = C * D * 2;
  constexpr int o_qp = 0, o_gv = o_qp + C * D * 2;
  constexpr int o_vs = o_gv + PK::ngate * 4, b1_bytes = o_vs + C * DVS * 2;
  constexpr int o_th = 0, o_aq = o_th + C * C * 2, b2_bytes = o_aq + C * C * 2;
  constexpr int b3_bytes = SCAL ? 16 : D * C * 2;
  __shared__ __attribute__((aligned(16))) char B1aS0[b1a_bytes];
  __shared__ __attribute__((aligned(16))) char B1aS1[b1a_bytes];
  __shared__ __attribute__((aligned(16))) char B1S0[b1_bytes];
  __shared__ __attribute__((aligned(16))) char B1S1[b1_bytes];
  __shared__ __attribute__((aligned(16))) char B2S0[b2_bytes];
  __shared__ __attribute__((aligned(16))) char B2S1[b2_bytes];
  __shared__ __attribute__((aligned(16))) char B3S0[b3_bytes];
  __shared__ __attribute__((aligned(16))) char B3S1[b3_bytes];
  // Written by the workgroup itself.
  // Written by the workgroup itself; swizzled like the packet tiles (see swz_key).
  __shared__ __attribute__((aligned(16))) _Float16 ST[DVS * D];  // S~^T
  __shared__ __attribute__((aligned(16))) _Float16 RT[DVS * C];  // R^T
  __shared__ __attribute__((aligned(16))) _Float16 DT[DVS * C];  // delta^T
  __shared__ __attribute__((aligned(16))) _Float16 DT2[SCAL ? DVS * C : 8];  // (Diag(e^{g_C - g}) delta)^T

  // Buffer set 0 or 1 (a compile-time choice, so that every access names its array).
  struct Set {
    _Float16* kp;
    _Float16* qp;
    _Float16* km;
    _Float16* th;
    _Float16* aq;
    float* gv;
    uint16_t* vs;  // bf16, as in v
  };
  auto set_of = [&](auto one) {
    constexpr bool B1 = decltype(one)::value;
    char* b1 = B1 ? B1S1 : B1S0;
    char* b2 = B1 ? B2S1 : B2S0;
    Set x;
    x.kp = reinterpret_cast<_Float16*>(B1 ? B1aS1 : B1aS0);
    x.qp = reinterpret_cast<_Float16*>(b1 + o_qp);
    x.gv = reinterpret_cast<float*>(b1 + o_gv);
    x.vs = reinterpret_cast<uint16_t*>(b1 + o_vs);
    x.th = reinterpret_cast<_Float16*>(b2 + o_th);
    x.aq = reinterpret_cast<_Float16*>(b2 + o_aq);
    x.km = reinterpret_cast<_Float16*>(B1 ? B3S1 : B3S0);
    return x;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int H = p.H;
  const WgRef wg = wg_ref(p);
  const int bh = wg.bh, h = bh % H;
  const int j0 = wg.slice * DVS;
  const SeqRef sq = seq_ref(p, bh, h);
  const int T = sq.len;  // this sequence's tokens
  const int nchunks = sq.nch;
  if (nchunks == 0) {
    pass_state(p, bh, j0, DVS);
    return;
  }
  const gptr<const char> pbase = opaque_gptr(ws) + sq.pkt0 * PK::bytes;
  const gptr<const char> vin = opaque_gptr(static_cast<const char*>(p.v));

  // State: wave w owns rows [16 w, 16 w + 16) x the DVS columns as NCT accumulator tiles
  // (lane: column 16 ct + l16, rows 16 w + 4 lg + r).
  f32x4 S[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = 16 * wave + 4 * lg + r;
      S[ct][r] = p.S0 ? p.S0[(int64_t(bh) * D + d) * D + j0 + 16 * ct + l16] : 0.f;
    }

  auto tok = [&](int t) { return (sq.tok0 + t) * H + h; };
  const int64_t tstride = int64_t(C) * H * D;  // elements between chunk c and c + 1
  // Besides two K+ and two Q+ copies, every wave issues one more 1 KB copy of batch 1, so that
  // all waves issue the same number and the partial waits are exact: wave w < ngv copies gate
  // block w, the next nvs waves the value slice, the rest gate block 0 again (same bytes, same
  // place).
  constexpr int ngv = PK::ngate * 4 / 1024, nvs = C * VU / 64;
  static_assert(ngv + nvs <= kScanWaves, "one extra copy per wave");
  const bool x_vs = wave >= ngv && wave < ngv + nvs;
  const int x_off = x_vs ? o_vs + 1024 * (wave - ngv) : o_gv + 1024 * (wave < ngv ? wave : 0);
  // value-slice unit of this thread (waves ngv .. ngv + nvs - 1): unit vu = 64 (wave - ngv) +
  // lane, token vu / VU, columns 8 (vu % VU) ..  The slice sits in LDS row-major with 16-byte
  // unit u of row r at u ^ vs_key(r), so that the transposing reads (8 rows per 32 lanes) are
  // conflict-free (with 64-byte rows, rows r and r + 4 share banks otherwise); this thread's
  // copy lands at unit vu % VU of row vt, so it fetches the unit stored there.
  auto vs_key = [](int r) { return VU == 4 ? ((r >> 2) & 1) << 1 : 0; };
  const int vu = (64 * (wave - ngv) + lane) & (C * VU - 1);
  const int vt = vu / VU, vc = 8 * ((vu % VU) ^ vs_key(vt));
  const int64_t v_off = tok(vt) * D + j0 + vc;
  const int64_t v_last = tok(T - 1) * D + j0 + vc;  // stands in for tokens past the end
  // Work split of the X and O stages.  With two value tiles (NCT == 2) wave w takes token rows
  // 16 (w % 4) and value tile w / 4 of both X_K (for R) and X_Q (for O), so every wave does the
  // same work; with one (NCT == 1) waves 0-3 take the X_K rows and waves 4-7 the X_Q rows.
  const int xct = NCT == 2 ? wave >> 2 : 0;
  const int64_t o_off = tok(16 * (wave & 3) + l16) * D + j0 + 16 * xct + 4 * lg;

  // Copies of chunk c's packet and value slice into buffer set X, plus the per-row decay
  // factors of this thread's state rows into registers.
  struct Fac {  // scalar decay: element 0 only
    float em[4], fc[4], fcm[4];
  };
  // Issued in three batches, each as early as its buffers are free and each waited for just
  // before its first reader: (1) key/query tiles, gate vector, values and factors, read from
  // the start of the chunk; (2) T and A_qk, read from the D stage on; (3) K^end (per-channel
  // decay), read by the state update.  Every wave issues the same number of loads in each
  // batch that a wait has to look past (past the last chunk the copies repeat the last chunk
  // into the idle set), so the number of loads a wave issues after each batch is known and a
  // partial vmcnt wait suffices.
  // Batch 1 goes out in parts: the K+ tile (read by the state update to the end of the chunk)
  // and the factors one chunk ahead, after the first barrier; the Q+ tile and the extra copy,
  // whose buffers are last read before the third barrier, with a per-head decay two chunks
  // ahead, right after that barrier, into the set of the chunk being processed; with a
  // per-channel decay the extra copy goes with K+ and the Q+ tile after the X stage's products
  // (each measured faster for its variant).
  constexpr bool kEarly = SCAL;
  auto fetch_q = [&](const Set& X, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(pk + PK::qp + 16 * tid + 8192 * i, reinterpret_cast<char*>(X.qp) + 1024 * wave + 8192 * i);
  };
  auto fetch_x = [&](const Set& X, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
    const bool ok = c * C + vt < T;
    const int64_t e = ok ? v_off + c * tstride : v_last;
    const gptr<const char> src = !x_vs ? pk + PK::gate + (x_off - o_gv) + 16 * lane
                                 : FG2  ? pk + PK::vt + 2 * (vt * D + j0 + vc)
                                        : vin + 2 * e;
    dma16(src, reinterpret_cast<char*>(X.qp) + x_off);
  };
  auto fetch_k = [&](const Set& X, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16(pk + PK::kp + 16 * tid + 8192 * i, reinterpret_cast<char*>(X.kp) + 1024 * wave + 8192 * i);
  };
  auto load_f = [&](Fac& F, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
    // the factors are loaded unconditionally (a conditional load would need a register copy,
    // and with it an immediate wait)
    const gptr<const float> gv = (gptr<const float>)(pk + PK::gate);
    if constexpr (SCAL) {
      F.em[0] = gv[GV_SC];
      F.fc[0] = gv[GV_SC + 1];
      F.fcm[0] = gv[GV_SC + 2];
    } else {
      const int d0 = 16 * wave + 4 * lg;
      const float4 a = gload_f4(gv, GV_EM + d0);
      const float4 bb = gload_f4(gv, GV_FC + d0);
      const float4 cc = gload_f4(gv, GV_FCM + d0);
      F.em[0] = a.x; F.em[1] = a.y; F.em[2] = a.z; F.em[3] = a.w;
      F.fc[0] = bb.x; F.fc[1] = bb.y; F.fc[2] = bb.z; F.fc[3] = bb.w;
      F.fcm[0] = cc.x; F.fcm[1] = cc.y; F.fcm[2] = cc.z; F.fcm[3] = cc.w;
    }
  };
  // the two parts of batch 1, each issued in one place: 1a after the first barrier (K+ with,
  // for a per-head decay, the factor loads; for a per-channel decay, the extra copy), 1b after
  // the third barrier (per-head decay: Q+ and the extra copy, two chunks ahead) or after the X
  // stage's products (per-channel decay: Q+ and the factor loads)
  auto fetch1a = [&](const Set& X, Fac& F, int c) {
    fetch_k(X, c);
    if constexpr (kEarly) load_f(F, c);
    else fetch_x(X, c);
  };
  auto fetch1b = [&](const Set& X, Fac& F, int c) {
    fetch_q(X, c);
    if constexpr (kEarly) fetch_x(X, c);
    else load_f(F, c);
  };
  // loads per lane of batches 1a, 1b and 3; batch 2 (below) has a lower bound for the scalar
  // decay, whose only wait past it is for batch 1a of the same chunk
  constexpr int kF = SCAL ? 1 : 3;
  constexpr int kB1a = kEarly ? 2 + kF : 3, kB1b = kEarly ? 3 : 2 + kF, kB2min = SCAL ? 1 : 2, kB3 = SCAL ? 0 : 2;
  // The twelve stored blocks of T and A_qk, 1 KB each: copy s (s = wave, and s = 8 + wave % 4
  // on waves 0-3, and with a per-channel decay also on waves 4-7, which repeat a copy so that
  // the count is exact for the wait on batch 3) takes stored block s % 6 of matrix s / 6 to LDS
  // block 2 I + H.
  auto fetch2 = [&](const Set& X, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
    auto copy = [&](int sl) {
      const int m = sl >= 6 ? 1 : 0, k = sl - 6 * m;
      const int lb = k < 2 ? 2 * k : k + 2;
      dma16(pk + PK::mat + 1024 * sl + 16 * lane, reinterpret_cast<char*>(X.th) + 8192 * m + 1024 * lb);
    };
    copy(wave);
    if (!SCAL || wave < 4) copy(8 + (wave & 3));
  };
  auto fetch3 = [&](const Set& X, int c) {
    if constexpr (!SCAL) {
      const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        dma16(pk + PK::kmt + 16 * tid + 8192 * i, reinterpret_cast<char*>(X.km) + 1024 * wave + 8192 * i);
    }
  };

  const int xrow = 16 * (wave & 3);
  const bool xq_wave = wave >= 4;
  // output tile of the previous chunk (every wave with NCT == 2, waves 4-7 otherwise), stored
  // one chunk later
  f32x4 OA;
  const bool o_wave = NCT == 2 || xq_wave;
  auto store_out = [&](int c, bool masked) {
    const int t = c * C + xrow + l16;
    if (!masked || t < T) store_o4(p.o, o_off + c * tstride, OA, p.o_bf16);
  };
  // With a per-head decay at 32-column slices the O tiles go out through LDS, so that each
  // store writes whole 128-byte rows (eight lanes per token) instead of two 64-byte halves from
  // two waves: the o stores cost the chunk less (a probe without them ran 12% faster).  Staged
  // O: [64 tokens][32 columns] fp32, 16-byte unit u of row t at u ^ (t % 8).  Wave w stores
  // tokens 8 w .. + 7; lane l token 8 w + l / 8, columns 4 (l % 8) .. + 3.
  constexpr bool kStage = SCAL && NCT == 2;
  __shared__ __attribute__((aligned(16))) float OS[kStage ? C * DVS : 4];
  const int s_t = 8 * wave + (lane >> 3), s_u = lane & 7;
  const int64_t s_off = tok(s_t) * D + j0 + 4 * s_u;
  // The row pieces are read from LDS after the first barrier and stored one chunk later, at the
  // start of the next step like the direct stores (a store issued after the chunk's factor loads
  // makes the compiler wait for all loads at the top of every chunk), alternating two registers
  // so that a piece is not overwritten right after its store.
  f32x4 SV[2];
  auto read_staged = [&](int k) { SV[k] = *reinterpret_cast<const f32x4*>(OS + s_t * DVS + 4 * (s_u ^ (s_t & 7))); };
  auto store_staged = [&](int k, int c, bool masked) {
    if (!masked || c * C + s_t < T) store_o4(p.o, s_off + c * tstride, SV[k], p.o_bf16);
  };

  Fac F;
  auto step = [&](int c, auto one) {
    constexpr bool B1 = decltype(one)::value;
    const Set X = set_of(Flag<B1>()), Y = set_of(Flag<!B1>());
    const int cn = c + 1 < nchunks ? c + 1 : c;  // chunk whose copies this step issues
    vm_wait<kB2min + kB3 + (kEarly ? kB1b : 0)>();  // batch 1 of this chunk, older stores
    if constexpr (!kStage) {
      if (c > 0 && o_wave) store_out(c - 1, false);
    } else {
      if (c > 1) store_staged(B1 ? 1 : 0, c - 2, false);  // read into SV[c % 2] two steps ago
    }
    float em[4], fC[4], fCm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      em[r] = F.em[SCAL ? 0 : r];
      fC[r] = F.fc[SCAL ? 0 : r];
      fCm[r] = F.fcm[SCAL ? 0 : r];
    }
    // S~^T = (Diag(em) S)^T, em = 1 (chunk-start reference)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      half4v hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(em[r] * S[ct][r]);
      *reinterpret_cast<half4v*>(ST + swz<16>(16 * ct + l16, 16 * wave + 4 * lg)) = hv;
    }
    lds_barrier();  // every wave's batch 1 of this chunk has landed; S~^T is complete
    if constexpr (kStage) {
      if (c > 0) read_staged(B1 ? 0 : 1);  // chunk c - 1 into SV[(c - 1) % 2]
    }
    fetch1a(Y, F, cn);

    // ---- X = [K+; Q+] S~ ------------------------------------------------------------------
    f32x4 XQ;  // X_Q^T tile of this wave's O rows (scaled), the start of O
    if constexpr (NCT == 2) {
      // Every LDS operand of the stage is read before the first product, so that the reads'
      // latencies overlap instead of adding up.  One S~ fragment set serves both products (A
      // and B fragments share their lane layout).
      half8 kf[4], qf[4], sf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = frag_s<16>(X.kp, xrow, 32 * ks, lane);
        qf[ks] = frag_s<16>(X.qp, xrow, 32 * ks, lane);
        sf[ks] = frag_s<16>(ST, 16 * xct, 32 * ks, lane);
      }
      // gates of rows xrow + 4 lg + r (X_K's layout) and of row xrow + l16 (X_Q^T's layout);
      // four consecutive floats in one read: a single address keeps the read's alias scope
      const float4 bt = *reinterpret_cast<const float4*>(X.gv + GV_BETA + xrow + 4 * lg);
      float4 fk = make_float4(1.f, 1.f, 1.f, 1.f);
      float fq = 1.f;
      if constexpr (SCAL) {
        fk = *reinterpret_cast<const float4*>(X.gv + GV_FP + xrow + 4 * lg);
        fq = X.gv[GV_FP + xrow + l16];
      }
      // v[xrow + 4 lg + r][16 xct + l16], r = 0..3, in one transposing read: lane 16 g + m
      // supplies row xrow + 4 g + m / 4, columns 16 xct + 4 (m % 4) .. + 3
      const int vr_row = xrow + 4 * lg + (l16 >> 2), vr_unit = 2 * xct + ((l16 & 3) >> 1);
      const short4v vr = ld_tr16(X.vs + vr_row * DVS + 8 * (vr_unit ^ vs_key(vr_row)) + 4 * (l16 & 1));
      f32x4 xk = {0.f, 0.f, 0.f, 0.f}, xq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        xk = mfma16x16x32(kf[ks], sf[ks], xk);  // rows: tokens xrow + 4 lg + r
        xq = mfma16x16x32(sf[ks], qf[ks], xq);  // transposed: token xrow + l16 is the column
      }
      if constexpr (!kEarly) {
        __builtin_amdgcn_sched_barrier(0);  // keeps the copies after the products
        fetch1b(Y, F, cn);
      }

      const float beta[4] = {bt.x, bt.y, bt.z, bt.w}, fkr[4] = {fk.x, fk.y, fk.z, fk.w};
      half4v hv;  // R = Diag(beta) (V - X_K), stored transposed
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = SCAL ? xk[r] * fkr[r] : xk[r];
        hv[r] = (_Float16)(beta[r] * (vval(uint16_t(vr[r])) - x));
        XQ[r] = SCAL ? xq[r] * fq : xq[r];
      }
      *reinterpret_cast<half4v*>(RT + swz<8>(16 * xct + l16, xrow + 4 * lg)) = hv;
    } else {
      f32x4 XR[NCT];
      // Every LDS operand of the stage is read, by every wave, before the first product, so
      // that the reads' latencies overlap instead of adding up.
      half8 af[4], bsv[NCT][4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // two reads and a choice of values, not a choice of pointers: LDS reads keep their
        // array's alias scope only through address arithmetic on one array, and without it every
        // read waits for the copies
        const half8 fk8 = frag_s<16>(X.kp, xrow, 32 * ks, lane), fq8 = frag_s<16>(X.qp, xrow, 32 * ks, lane);
        af[ks] = xq_wave ? fq8 : fk8;
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bsv[ct][ks] = frag_s<16>(ST, 16 * ct, 32 * ks, lane);
      // gates of rows xrow + 4 lg + r (X_K's layout) and of row xrow + l16 (X_Q^T's layout);
      // four consecutive floats in one read: a single address keeps the read's alias scope
      // (per-element addresses would lose it and then wait for the copies)
      const float4 bt = *reinterpret_cast<const float4*>(X.gv + GV_BETA + xrow + 4 * lg);
      float4 fk = make_float4(1.f, 1.f, 1.f, 1.f);
      float fq = 1.f;
      if constexpr (SCAL) {
        fk = *reinterpret_cast<const float4*>(X.gv + GV_FP + xrow + 4 * lg);
        fq = X.gv[GV_FP + xrow + l16];
      }
      // v[xrow + 4 lg + r][16 ct + l16], r = 0..3, in one transposing read per column tile:
      // lane 16 g + m supplies row xrow + 4 g + m / 4, columns 16 ct + 4 (m % 4) .. + 3
      short4v vr[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int vr_row = xrow + 4 * lg + (l16 >> 2), vr_unit = 2 * ct + ((l16 & 3) >> 1);
        vr[ct] = ld_tr16(X.vs + vr_row * DVS + 8 * (vr_unit ^ vs_key(vr_row)) + 4 * (l16 & 1));
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          // the wave-dependent operand order is a choice of operands for one product: two
          // products behind a branch gave wrong results in one register allocation
          const half8 opa = xq_wave ? bsv[ct][ks] : af[ks], opb = xq_wave ? af[ks] : bsv[ct][ks];
          acc = mfma16x16x32(opa, opb, acc);
        }
        if constexpr (SCAL) {
          // rows of X_K are tokens xrow + 4 lg + r; X_Q^T has token xrow + l16 as its column
          acc[0] *= xq_wave ? fq : fk.x;
          acc[1] *= xq_wave ? fq : fk.y;
          acc[2] *= xq_wave ? fq : fk.z;
          acc[3] *= xq_wave ? fq : fk.w;
        }
        XR[ct] = acc;
      }
      if constexpr (!kEarly) {
        __builtin_amdgcn_sched_barrier(0);  // keeps the copies after the products
        fetch1b(Y, F, cn);
      }

      if (!xq_wave) {
        // R = Diag(beta) (V - X_K), stored transposed
        const float beta[4] = {bt.x, bt.y, bt.z, bt.w};
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          half4v hv;
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(beta[r] * (vval(uint16_t(vr[ct][r])) - XR[ct][r]));
          *reinterpret_cast<half4v*>(RT + swz<8>(16 * ct + l16, xrow + 4 * lg)) = hv;
        }
      }
      XQ = XR[0];
    }
    vm_wait<kB3 + kB1b + kB1a>();  // batch 2 of this chunk
    lds_barrier();
    // Checkpoint stores go out right after a wait, so that they have the stages up to the next wait
    // to complete (a partial wait also waits for every store issued before it); S still holds the
    // chunk's incoming state until the S stage.
    if constexpr (CKPT) store_state_h(static_cast<_Float16*>(p.ck_S) + (sq.pkt0 + c) * D * D, j0, S);
    fetch2(Y, cn);

    // ---- D: delta = T R, stored transposed ---------------------------------------------
    static_assert(4 * NCT <= kScanWaves, "one delta tile per wave");
    f32x4 dck;  // this wave's delta tile (wave < 4 NCT), for the checkpoint
#pragma unroll
    for (int n = wave; n < 4 * NCT; n += kScanWaves) {
      const int i = n & 3, ct = n >> 2;
      // T is lower triangular with zero upper tiles in the packet, so the products run over
      // both halves unconditionally (no branch around the reads)
      half8 ta[2], rb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ta[ks] = frag_tri(X.th, i, ks, lane);
        rb[ks] = frag_s<8>(RT, 16 * ct, 32 * ks, lane);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma16x16x32(ta[ks], rb[ks], acc);
      half4v hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = (_Float16)acc[r];
      *reinterpret_cast<half4v*>(DT + swz<8>(16 * ct + l16, 16 * i + 4 * lg)) = hv;
      dck = acc;
      if constexpr (SCAL) {
        // K^end^T delta = k^T (Diag(e^{g_C - g}) delta): the state update takes the scaled copy
        const float4 fm = *reinterpret_cast<const float4*>(X.gv + GV_FM + 16 * i + 4 * lg);
        hv[0] = (_Float16)(acc[0] * fm.x);
        hv[1] = (_Float16)(acc[1] * fm.y);
        hv[2] = (_Float16)(acc[2] * fm.z);
        hv[3] = (_Float16)(acc[3] * fm.w);
        *reinterpret_cast<half4v*>(DT2 + swz<8>(16 * ct + l16, 16 * i + 4 * lg)) = hv;
      }
    }
    if constexpr (!SCAL) vm_wait<kB1b + kB1a + kB2min>();  // batch 3 of this chunk
    lds_barrier();
    if constexpr (CKPT) {  // delta, after the wait (see the state's checkpoint above)
      if (wave < 4 * NCT) store_rows(p.ck_M, sq.pkt0 + c, 16 * (wave & 3) + 4 * lg, j0 + 16 * (wave >> 2) + l16, dck);
    }
    fetch3(Y, cn);
    if constexpr (kEarly) fetch1b(X, F, c + 2 < nchunks ? c + 2 : nchunks - 1);  // c + 2 uses set X

    // ---- O: rows xrow .. + 15, value tile xct (stored with the next chunk) -----------------
    if (o_wave) {
      const int i = wave & 3;
      // A_qk has zero upper tiles in the packet: both halves, no branch
      half8 qa[2], db[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qa[ks] = frag_tri(X.aq, i, ks, lane);
        db[ks] = frag_s<8>(DT, 16 * xct, 32 * ks, lane);
      }
      f32x4 acc = XQ;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc = mfma16x16x32(db[ks], qa[ks], acc);
      OA = acc;
      if constexpr (kStage) {
        const int t = xrow + l16, u = 4 * xct + lg;
        *reinterpret_cast<f32x4*>(OS + t * DVS + 4 * (u ^ (t & 7))) = acc;
      }
    }

    // ---- S: state update for this wave's rows ---------------------------------------------
    {
      f32x4 acc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      half8 ak[2], dk[NCT][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ak[ks] = frag_ts(SCAL ? X.kp : X.km, 16 * wave, 32 * ks, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) dk[ct][ks] = frag_s<8>(SCAL ? DT2 : DT, 16 * ct, 32 * ks, lane);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] = mfma16x16x32(ak[ks], dk[ct][ks], acc[ct]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[ct][r] = fmaf(fC[r], S[ct][r], fCm[r] * acc[ct][r]);
    }
    // No barrier here: the next step's first LDS write (S~^T) targets a tile last read before
    // this step's second barrier, and its copies go out only after its own first barrier.
  };

  // The upper blocks (0,1) and (1,1) of T and A_qk, in both buffer sets, are zero and never
  // copied; written before the first copy, so that no write waits for one.
  if (tid < 256) {
    const int zb = o_th + 8192 * ((tid >> 6) & 1) + 1024 * (1 + 2 * (tid >> 7)) + 16 * lane;
    const uint4 zz = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(B2S0 + zb) = zz;
    *reinterpret_cast<uint4*>(B2S1 + zb) = zz;
  }
  if constexpr (kEarly) fetch1b(set_of(Flag<false>()), F, 0);
  fetch1a(set_of(Flag<false>()), F, 0);
  if constexpr (!kEarly) fetch1b(set_of(Flag<false>()), F, 0);
  fetch2(set_of(Flag<false>()), 0);
  fetch3(set_of(Flag<false>()), 0);
  if constexpr (kEarly) fetch1b(set_of(Flag<true>()), F, nchunks > 1 ? 1 : 0);
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(c, Flag<false>());
    step(c + 1, Flag<true>());
  }
  if (c < nchunks) step(c, Flag<false>());
  vm_wait_all();
  if constexpr (kStage) {
    // chunk nchunks - 2 was read in the last step; chunk nchunks - 1 is still in LDS
    if (nchunks > 1) store_staged(nchunks & 1, nchunks - 2, false);
    lds_barrier();
    read_staged((nchunks - 1) & 1);
    store_staged((nchunks - 1) & 1, nchunks - 1, true);
  } else {
    if (o_wave) store_out(nchunks - 1, true);
  }

  if (p.S_T) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * wave + 4 * lg + r;
        p.S_T[(int64_t(bh) * D + d) * D + j0 + 16 * ct + l16] = S[ct][r];
      }
  }
}

// ------------------------------------------------------------------------------------------
// Adjoint scan (gradients): the chunks of one (b, h, value slice) from the last, carrying the
// state's adjoint G = dL/dS at the end of the chunk in fp32 registers like the forward state.
// Reversing the chunk form above (L = sum(o * dO) + sum(S_T * dS_T)), one chunk maps G to the
// adjoint at its start,
//   X1 = W1^T dO + E G~,  Z = -B T^T X1,  G <- Diag(e^{g_C}) G + Q+^T dO + K+^T Z,
// with W1 = A_qk, E = K^end, B = Diag(beta) for symmetric gates (X1 is delta's adjoint, Z the
// adjoint of K+ S) and W1 = A_qu, E = U^end, B = I for general gates (X1 = -M's adjoint).  With a
// per-head decay the packet holds plain k and q: K^end = Diag(e^{g_C - g}) k scales the rows of
// k G~, and Q+ = Diag(e^{g}) q, K+ = Diag(e^{g}) k put e^{g_t} on dO's and Z's rows.  The
// adjoint at the end of every chunk goes to p.ck_G (the chunk-parallel adjoint of the token
// loop starts there), and the one at the start of the sequence is dS0.  Eight waves, register
// staging one chunk ahead, four barriers per chunk.
// ------------------------------------------------------------------------------------------
template <bool DCH, bool GEN, bool FG2, int DVS>
__global__ __launch_bounds__(kScanThreads) void chunk_adjoint_scan_kernel(Problem p, const char* __restrict__ ws,
                                                                          const float* __restrict__ dO,
                                                                          const float* __restrict__ dS_T,
                                                                          float* __restrict__ dS0) {
  using PK = Packet<DCH, GEN, FG2>;
  constexpr bool SCAL = !DCH && !GEN;
  constexpr int NCT = DVS / 16;
  constexpr int VPT = DVS / 8;       // dO columns per thread in its load
  constexpr int W1 = GEN ? 3 : 1;    // packet matrix of W1
  // LDS: operand tiles (the packet's swizzled layout), T and W1 as eight 16 x 32 blocks each,
  // the gate vector, and the workgroup's own G~^T, dO^T (and Diag(e^g) dO^T), X1^T, Z^T
  __shared__ __attribute__((aligned(16))) _Float16 QP[C * D];
  __shared__ __attribute__((aligned(16))) _Float16 KP[C * D];
  __shared__ __attribute__((aligned(16))) _Float16 EP[SCAL ? 8 : C * D];
  __shared__ __attribute__((aligned(16))) _Float16 TM[2 * 8 * 512];  // T, then W1
  __shared__ __attribute__((aligned(16))) float GV[PK::ngate];
  __shared__ __attribute__((aligned(16))) _Float16 GT[DVS * D];
  __shared__ __attribute__((aligned(16))) _Float16 DOT[DVS * C];
  __shared__ __attribute__((aligned(16))) _Float16 DOG[SCAL ? DVS * C : 8];
  __shared__ __attribute__((aligned(16))) _Float16 X1T[DVS * C];
  __shared__ __attribute__((aligned(16))) _Float16 ZT[DVS * C];
  const _Float16* const EE = SCAL ? KP : EP;  // E's rows: K^end (or k, scaled), U^end

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int H = p.H;
  const WgRef wg = wg_ref(p);
  const int bh = wg.bh, h = bh % H;
  const int j0 = wg.slice * DVS;
  const SeqRef sq = seq_ref(p, bh, h);
  const int T = sq.len;
  const int nchunks = sq.nch;
  const gptr<const char> pbase = opaque_gptr(ws) + sq.pkt0 * PK::bytes;
  const gptr<const float> dOin = opaque_gptr(dO);

  // G: wave w owns rows [16 w, 16 w + 16) x the DVS columns (lane: column 16 ct + l16, rows
  // 16 w + 4 lg + r)
  f32x4 G[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = 16 * wave + 4 * lg + r;
      G[ct][r] = dS_T ? dS_T[(int64_t(bh) * D + d) * D + j0 + 16 * ct + l16] : 0.f;
    }
  if (nchunks == 0) {
    if (dS0) store_state(dS0 + int64_t(bh) * D * D, j0, G);
    return;
  }
  // zero upper blocks (0,1) and (1,1) of both matrices, never copied
  if (tid < 256) *reinterpret_cast<uint4*>(TM + 4096 * (tid >> 7) + 512 * (1 + 2 * ((tid >> 6) & 1)) + 8 * lane) =
      make_uint4(0, 0, 0, 0);

  auto tok = [&](int t) { return (sq.tok0 + t) * H + h; };
  const int vtok = tid >> 3, vcol = (tid & 7) * VPT;  // dO slice: token tid / 8
  const int64_t tstride = int64_t(C) * H * D;
  const int64_t d_off = tok(vtok) * D + j0 + vcol, d_last = tok(T - 1) * D + j0 + vcol;

  struct Pref {
    uint4 tl[SCAL ? 4 : 6];  // Q+, K+ (, E) units tid and tid + 512
    uint4 mr[2];             // stored blocks of T and W1: units tid, tid + 512 (< 768)
    float4 gv;               // gate vector floats 4 tid .. (tid < ngate / 4)
    float dv[VPT];           // dO (rows past the last token hold the last token's, masked at use)
    bool ok;                 // this thread's token lies inside the sequence
  };
  auto load = [&](Pref& P, int c) {
    const gptr<const char> pk = pbase + int64_t(c) * PK::bytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      P.tl[i] = ldb16(pk, PK::qp + 16 * (tid + kScanThreads * i));
      P.tl[2 + i] = ldb16(pk, PK::kp + 16 * (tid + kScanThreads * i));
      if constexpr (!SCAL) P.tl[4 + i] = ldb16(pk, (GEN ? PK::umt : PK::kmt) + 16 * (tid + kScanThreads * i));
    }
    // every load unconditional (units past the stored ones repeat the last), so that no load sits
    // in a branch and each is waited for only where it is used
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int u = min(tid + kScanThreads * j, 767), m = u / 384, k = (u % 384) / 64;
      P.mr[j] = ldb16(pk, PK::mat + (m ? W1 : 0) * PK::matb + 1024 * k + 16 * (u % 64));
    }
    P.gv = ldf16(pk, PK::gate + 16 * min(tid, PK::ngate / 4 - 1));
    P.ok = c * C + vtok < T;
    const int64_t e = P.ok ? d_off + c * tstride : d_last;
#pragma unroll
    for (int i = 0; i < VPT; i += 2) {
      const f32x2 x = *(gptr<const f32x2>)(dOin + e + i);
      P.dv[i] = x.x;
      P.dv[i + 1] = x.y;
    }
  };

  // scale of the rows of Z (and of E G~ with a per-head decay): the chunk's per-row factors
  const int zi = 16 * (wave & 3) + 4 * lg;  // rows of this wave's X1 / Z tile
  const int zct = NCT == 2 ? wave >> 2 : 0;
  const bool zwave = NCT == 2 || wave < 4;

  // Checkpoint stores go out right after the chunk's one wait for its staged loads (in the L stage),
  // so that they have the whole chunk to complete before the next one (a wait for a load also waits
  // for every store issued before it): G at the chunk end (G still holds it until the update), and
  // the previous step's Z, held in registers until then.
  f32x4 zpend = {0.f, 0.f, 0.f, 0.f};
  int zpend_c = -1;
  auto store_z = [&](int cz) {
    if (zwave) store_rows(p.ck_Z, sq.pkt0 + cz, zi, j0 + 16 * zct + l16, zpend);
  };
  auto step = [&](int c, Pref& P) {
    // ---- L: the chunk's packet, dO^T and G~^T into LDS ------------------------------------
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + kScanThreads * i;
      *reinterpret_cast<uint4*>(QP + 8 * u) = P.tl[i];
      *reinterpret_cast<uint4*>(KP + 8 * u) = P.tl[2 + i];
      if constexpr (!SCAL) *reinterpret_cast<uint4*>(EP + 8 * u) = P.tl[4 + i];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int u = tid + kScanThreads * j, m = u / 384, k = (u % 384) / 64;
      const int lb = k < 2 ? 2 * k : k + 2;
      if (u < 768) *reinterpret_cast<uint4*>(TM + 4096 * m + 512 * lb + 8 * (u % 64)) = P.mr[j];
    }
    if (tid < PK::ngate / 4) *reinterpret_cast<float4*>(GV + 4 * tid) = P.gv;
#pragma unroll
    for (int i = 0; i < VPT; ++i) DOT[swz<8>(vcol + i, vtok)] = (_Float16)(P.ok ? P.dv[i] : 0.f);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      *reinterpret_cast<half4v*>(GT + swz<16>(16 * ct + l16, 16 * wave + 4 * lg)) = cvt4(G[ct]);
    lds_barrier();
    store_state_h(static_cast<_Float16*>(p.ck_G) + (sq.pkt0 + c) * D * D, j0, G);
    if (zpend_c >= 0) store_z(zpend_c);
    if constexpr (SCAL) {  // Diag(e^{g}) dO^T for Q+^T dO
#pragma unroll
      for (int i = 0; i < VPT; ++i) DOG[swz<8>(vcol + i, vtok)] = (_Float16)((P.ok ? P.dv[i] : 0.f) * GV[GV_FP + vtok]);
    }
    const int cn = c > 0 ? c - 1 : 0;
    load(P, cn);

    // ---- X1 = W1^T dO + E G~, stored transposed --------------------------------------------
    if (zwave) {
      const int I = wave & 3;
      f32x4 xa = {0.f, 0.f, 0.f, 0.f}, xb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        xa = mfma16x16x32(frag_tri_t(TM + 4096, 16 * I, 32 * ks, lane), frag_s<8>(DOT, 16 * zct, 32 * ks, lane), xa);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        xb = mfma16x16x32(frag_s<16>(EE, 16 * I, 32 * ks, lane), frag_s<16>(GT, 16 * zct, 32 * ks, lane), xb);
      half4v hv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float eb = SCAL ? GV[GV_FM + zi + r] : 1.f;  // K^end = Diag(e^{g_C - g}) k
        hv[r] = (_Float16)(fmaf(eb, xb[r], xa[r]));
      }
      *reinterpret_cast<half4v*>(X1T + swz<8>(16 * zct + l16, zi)) = hv;
    }
    lds_barrier();
    // ---- Z = -B T^T X1 (per-head decay: times Diag(e^{g})), stored transposed ---------------
    if (zwave) {
      const int I = wave & 3;
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        z = mfma16x16x32(frag_tri_t(TM, 16 * I, 32 * ks, lane), frag_s<8>(X1T, 16 * zct, 32 * ks, lane), z);
      half4v hv;
      f32x4 zu;  // Z itself (without the per-head decay's row factor)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float f = GEN ? -1.f : -GV[GV_BETA + zi + r];
        zu[r] = f * z[r];
        if constexpr (SCAL) f *= GV[GV_FP + zi + r];
        hv[r] = (_Float16)(f * z[r]);
      }
      *reinterpret_cast<half4v*>(ZT + swz<8>(16 * zct + l16, zi)) = hv;
      zpend = zu;
    }
    zpend_c = c;
    lds_barrier();
    // ---- G <- Diag(e^{g_C}) G + Q+^T dO + K+^T Z (this wave's rows) -------------------------
    {
      f32x4 acc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const half8 aq = frag_ts(QP, 16 * wave, 32 * ks, lane), ak = frag_ts(KP, 16 * wave, 32 * ks, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          acc[ct] = mfma16x16x32(aq, frag_s<8>(SCAL ? DOG : DOT, 16 * ct, 32 * ks, lane), acc[ct]);
          acc[ct] = mfma16x16x32(ak, frag_s<8>(ZT, 16 * ct, 32 * ks, lane), acc[ct]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float fC = SCAL ? GV[GV_SC + 1] : GV[GV_FC + 16 * wave + 4 * lg + r];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) G[ct][r] = fmaf(fC, G[ct][r], acc[ct][r]);
      }
    }
    lds_barrier();
  };

  Pref PA;
  load(PA, nchunks - 1);
  for (int c = nchunks - 1; c >= 0; --c) step(c, PA);
  if (zpend_c >= 0) store_z(zpend_c);
  if (dS0) store_state(dS0 + int64_t(bh) * D * D, j0, G);
}

template <bool DCH, bool GEN, bool FG2>
hipError_t launch_adjoint_scan(const Problem& p, const char* ws, const float* dO, const float* dS_T, float* dS0,
                               hipStream_t stream) {
  const int64_t bh = int64_t(p.B) * p.H;
  if (bh >= 64) {
    dim3 grid(unsigned(bh), unsigned(D / 32));
    hipLaunchKernelGGL((chunk_adjoint_scan_kernel<DCH, GEN, FG2, 32>), grid, dim3(kScanThreads), 0, stream, p, ws,
                       dO, dS_T, dS0);
  } else {
    dim3 grid(unsigned(bh), unsigned(D / 16));
    hipLaunchKernelGGL((chunk_adjoint_scan_kernel<DCH, GEN, FG2, 16>), grid, dim3(kScanThreads), 0, stream, p, ws,
                       dO, dS_T, dS0);
  }
  return hipGetLastError();
}

template <bool DCH, int DVS, bool FG2>
hipError_t launch_scan_sym(const Problem& p, const char* ws, hipStream_t stream) {
  dim3 grid(unsigned(p.B * p.H), unsigned(D / DVS));
  if (p.ck_S)
    hipLaunchKernelGGL((chunk_scan_sym_kernel<DCH, DVS, FG2, true>), grid, dim3(kScanThreads), 0, stream, p, ws);
  else
    hipLaunchKernelGGL((chunk_scan_sym_kernel<DCH, DVS, FG2>), grid, dim3(kScanThreads), 0, stream, p, ws);
  return hipGetLastError();
}

template <bool DCH, int DVS>
hipError_t launch_scan_gen(const Problem& p, const char* ws, hipStream_t stream) {
  dim3 grid(unsigned(p.B * p.H), unsigned(D / DVS));
  if (p.ck_S) {
    if (p.write_channel)
      hipLaunchKernelGGL((chunk_scan_kernel<DCH, true, true, DVS, true>), grid, dim3(kScanThreads), 0, stream, p, ws);
    else
      hipLaunchKernelGGL((chunk_scan_kernel<DCH, true, false, DVS, true>), grid, dim3(kScanThreads), 0, stream, p, ws);
  } else if (p.write_channel) {
    hipLaunchKernelGGL((chunk_scan_kernel<DCH, true, true, DVS>), grid, dim3(kScanThreads), 0, stream, p, ws);
  } else {
    hipLaunchKernelGGL((chunk_scan_kernel<DCH, true, false, DVS>), grid, dim3(kScanThreads), 0, stream, p, ws);
  }
  return hipGetLastError();
}

int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }

template <bool DCH, bool GEN, bool FG2 = false>
hipError_t launch_variant(const Problem& p, void* workspace, hipStream_t stream) {
  const int nchunks = (p.T + C - 1) / C;
  char* ws = static_cast<char*>(workspace);
  // packed sequences: the grid is sized for the most chunks their lengths allow; the kernel
  // reads the actual count from the table
  const int64_t nblk = p.chunks ? int64_t(p.H) * varlen_max_chunks(p.B, p.T) : int64_t(p.B) * p.H * nchunks;
  // Persistent: as many workgroups as fit at once (two per compute unit), each walking every
  // grid-th chunk with its next chunk's inputs in flight.
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const int64_t resident = int64_t(ncu) * 2;
  const int64_t grid = nblk < resident ? nblk : resident;
  if constexpr (!DCH && !GEN)
    hipLaunchKernelGGL((chunk_prep_scalar_kernel<FG2>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p, ws, nchunks,
                       nblk);
  else
    hipLaunchKernelGGL((chunk_prep_ch_kernel<DCH, GEN, FG2>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p, ws,
                       nchunks, nblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Fill the 256 compute units with (b, h, value-slice) workgroups while keeping the slices
  // (each stages its chunk's operand tiles) as wide as that allows.
  const int64_t bh = int64_t(p.B) * p.H;
  if constexpr (GEN) {
    // a dense batch: the full-width segmented scan (one workgroup per (b, h, segment) with all
    // value columns), its segment maps after the packets
    if (!p.chunks)
      return launch_scan_wide(p, ws, reinterpret_cast<float*>(ws + round256(int64_t(p.B) * p.H * nchunks *
                                                                              Packet<DCH, GEN>::bytes)),
                              stream);
    return bh >= 64 ? launch_scan_gen<DCH, 32>(p, ws, stream) : launch_scan_gen<DCH, 16>(p, ws, stream);
  } else {
    return bh >= 64 ? launch_scan_sym<DCH, 32, FG2>(p, ws, stream) : launch_scan_sym<DCH, 16, FG2>(p, ws, stream);
  }
}

int64_t packet_bytes(bool symmetric, bool decay_channel, bool rate_sqrt) {
  if (rate_sqrt) return decay_channel ? Packet<true, false, true>::bytes : Packet<false, false, true>::bytes;
  return !symmetric ? Packet<true, true>::bytes : decay_channel ? Packet<true, false>::bytes : Packet<false, false>::bytes;
}

}  // namespace

size_t chunk128_workspace_bytes(int B, int T, int H, bool symmetric, bool decay_channel, bool rate_sqrt) {
  const int64_t nchunks = (int64_t(T) + C - 1) / C;
  const int64_t packets = int64_t(B) * H * nchunks * packet_bytes(symmetric, decay_channel, rate_sqrt);
  // general gates: the full-width scan's segment maps and entering states follow the packets
  if (!symmetric && !rate_sqrt) return size_t(round256(packets) + int64_t(wide_workspace_bytes(B, T, H)));
  return size_t(packets);
}

// Packed sequences: packets of at most varlen_max_chunks chunks per head, then the chunk
// table, the sequence table, the sequence order and the chunk count.
size_t chunk128_varlen_workspace_bytes(int nseq, int T, int H, bool symmetric, bool decay_channel, bool rate_sqrt) {
  const int64_t maxc = varlen_max_chunks(nseq, T);
  return size_t(int64_t(H) * maxc * packet_bytes(symmetric, decay_channel, rate_sqrt) + round256(maxc * 16) +
                round256(int64_t(nseq) * 16) + round256(int64_t(nseq) * 4) + 256);
}

void chunk128_varlen_tables(Problem& p, void* workspace) {
  const int64_t maxc = varlen_max_chunks(p.B, p.T);
  char* tables = static_cast<char*>(workspace) +
                 int64_t(p.H) * maxc * packet_bytes(p.symmetric, p.decay_channel, p.rate_sqrt);
  p.chunks = reinterpret_cast<int4*>(tables);
  p.seqs = reinterpret_cast<int4*>(tables + round256(maxc * 16));
  int* order = reinterpret_cast<int*>(tables + round256(maxc * 16) + round256(int64_t(p.B) * 16));
  p.order = order;
  p.nchunks_total = order + round256(int64_t(p.B) * 4) / 4;
}

hipError_t launch_chunk128_varlen(Problem p, const int* cu, void* workspace, hipStream_t stream) {
  chunk128_varlen_tables(p, workspace);
  hipError_t e = launch_varlen_setup(cu, p.B, p.T, p.H, C, const_cast<int4*>(p.seqs), const_cast<int4*>(p.chunks),
                                     const_cast<int*>(p.nchunks_total), const_cast<int*>(p.order), stream);
  if (e != hipSuccess) return e;
  return launch_chunk128(p, workspace, stream);
}

hipError_t launch_chunk128_adjoint(const Problem& p, const void* workspace, const float* dO, const float* dS_T,
                                   float* dS0, hipStream_t stream) {
  const char* ws = static_cast<const char*>(workspace);
  if (!p.symmetric && !p.rate_sqrt && !p.chunks) {
    // separate erase and write gates over a dense batch: the full-width segmented adjoint scan,
    // its segment maps where the forward's were (after the packets)
    const int64_t nchunks = (int64_t(p.T) + C - 1) / C;
    float* extra = reinterpret_cast<float*>(const_cast<char*>(ws) +
                                            round256(int64_t(p.B) * p.H * nchunks * Packet<true, true>::bytes));
    return launch_adjoint_wide(p, ws, extra, dO, dS_T, dS0, stream);
  }
  if (p.rate_sqrt)
    return p.decay_channel ? launch_adjoint_scan<true, false, true>(p, ws, dO, dS_T, dS0, stream)
                           : launch_adjoint_scan<false, false, true>(p, ws, dO, dS_T, dS0, stream);
  if (p.decay_channel)
    return p.symmetric ? launch_adjoint_scan<true, false, false>(p, ws, dO, dS_T, dS0, stream)
                       : launch_adjoint_scan<true, true, false>(p, ws, dO, dS_T, dS0, stream);
  return p.symmetric ? launch_adjoint_scan<false, false, false>(p, ws, dO, dS_T, dS0, stream)
                     : launch_adjoint_scan<false, true, false>(p, ws, dO, dS_T, dS0, stream);
}

hipError_t launch_chunk128(const Problem& p, void* workspace, hipStream_t stream) {
  if (p.rate_sqrt)  // FG2's per-channel rate keeps the symmetric gates
    return p.decay_channel ? launch_variant<true, false, true>(p, workspace, stream)
                           : launch_variant<false, false, true>(p, workspace, stream);
  const bool symmetric = p.symmetric;
  if (p.decay_channel)
    return symmetric ? launch_variant<true, false>(p, workspace, stream)
                     : launch_variant<true, true>(p, workspace, stream);
  return symmetric ? launch_variant<false, false>(p, workspace, stream)
                   : launch_variant<false, true>(p, workspace, stream);
}

}  // namespace dr
