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
// per-channel reference gm (g at the chunk midpoint):
//   K+ = k e^{g - gm}, Q+ = q e^{g - gm}, K- = k e^{gm - g}, U- = (e * k) e^{gm - g}
//   A_kk = strict_lower(K+ K-^T)  A_ku = strict_lower(K+ U-^T)  A_qk = lower(Q+ K-^T)
//   A_qu = lower(Q+ U-^T)          X_K = K+ S~,  X_Q = Q+ S~,  S~ = Diag(e^{gm}) S
// symmetric gates (one beta for erase and write):
//   T = (I + Diag(beta) A_kk)^{-1},  delta = T Diag(beta) (V - X_K)
//   O = X_Q + A_qk delta,            S <- Diag(e^{g_C}) S + Diag(e^{g_C - gm}) K-^T delta
// general gates (erase e, write w; Vt = w * v):
//   T = (I + A_ku)^{-1},  M = T (X_K + A_kk Vt)
//   O = X_Q + A_qk Vt - A_qu M,  S <- Diag(e^{g_C}) S + Diag(e^{g_C - gm}) (K-^T Vt - U-^T M)
//
// Two kernels.  chunk_prep_kernel runs one workgroup per chunk (all chunks of all heads in
// parallel) and writes everything that does not depend on the state into a per-chunk packet
// in the caller's workspace: T (the only factor that needs a serial algorithm), the Gram
// matrices, the gate factors and, unless the decay is one scalar per token, the decayed fp16
// operand tiles K+, Q+, K-^T (and U-^T).  chunk_scan_kernel then walks the chunks of one
// (b, h, value slice) in order, carrying the fp32 state in registers; per chunk it copies the
// packet into LDS and runs only the state-dependent products, so no exponential, prefix sum
// or format conversion is repeated by the value slices of a head.  With a scalar decay the
// packet holds no decayed tiles: it carries the plain k and q, and the scan applies the
// per-token factors e^{+-(g_t - gm)} to product rows instead.
//
// FG2-GDN's per-channel rate beta runs the symmetric kernels on the scaled pair
// (sqrt(beta) k, sqrt(beta) v) with a unit gate: the prep scales k as it loads it and writes the
// scaled values into the packet, from where the scan copies its value slice.  Packed sequences
// of different lengths run the same kernels over tables of their chunks (prep) and sequences
// (scan), written into the workspace by a set-up kernel.
//
// Products use v_mfma_f32_16x16x32_f16 (fp16 operands, fp32 accumulation).  Gram tiles are
// computed transposed (A^T = K- Q+^T) so that each lane owns four consecutive columns of one
// row of A and stores them with one vector write.
//
// Range: the midpoint reference keeps every fp16 operand within e^{+-(half-chunk decay)}.  The
// exponents are clamped at 11 (e^11 < 65504), so a per-channel log-decay sum below -11 over half
// a chunk loses accuracy (the token-by-token path has no such limit).

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int C = 64;      // chunk length
constexpr int D = 128;     // dk == dv
constexpr int KS = 136;    // row stride (halves) of [64][128] tiles: 16-byte pad
constexpr int CS = 72;     // row stride (halves) of [*][64] tiles
constexpr int AFS = 68;    // row stride (floats) of the fp32 64 x 64 matrix (16-byte rows)
constexpr int kThreads = 256;
constexpr float kExpClamp = 11.f;

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

__device__ __forceinline__ f32x4 mfma16(half4v a, half4v b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 cvt8(const float* x) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)x[i];
  return h;
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 u, float* f) {
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}

__device__ __forceinline__ float clamped_exp(float x) { return __expf(fminf(x, kExpClamp)); }

__device__ __forceinline__ void unpack8(float4 a, float4 b, float* f) {
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// 16 bytes at byte offset `off` of a global byte pointer.
__device__ __forceinline__ uint4 ldb16(gptr<const char> base, int64_t off) {
  const u32x4 x = *(gptr<const u32x4>)(base + off);
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ float4 ldf16(gptr<const char> base, int64_t off) {
  const f32x4 x = *(gptr<const f32x4>)(base + off);
  return make_float4(x.x, x.y, x.z, x.w);
}

// Chunk-local inclusive prefix sums of the log-decay.  Thread (token quad tg, channel octet
// d8) holds its 4 x 8 (per channel) or 4 (per head: wave 0 lane t holds token t) log-decays;
// on return g[r][ch] (per head: g[r][0]) is the cumulative log-decay of its tokens and GSC holds
// per-wave totals (per channel, [4][128]) or the 64 per-token prefixes (per head).
template <bool DCH>
__device__ __forceinline__ void chunk_cumsum(const float (&ldr)[DCH ? 4 : 1][DCH ? 8 : 1], float lds,
                                             float (&g)[4][DCH ? 8 : 1], float* GSC, int tid) {
  const int lane = tid & 63, wave = tid >> 6, lg = lane >> 4, d8 = tid & 15, tg = tid >> 4;
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
    lds_barrier();
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
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 4; ++r) g[r][0] = GSC[4 * tg + r];
  }
}

template <bool DCH>
__device__ __forceinline__ float chunk_gmid(const float* GSC, int d) {
  return DCH ? GSC[d] + GSC[D + d] : GSC[31];
}

template <bool DCH>
__device__ __forceinline__ float chunk_gend(const float* GSC, int d) {
  return DCH ? GSC[d] + GSC[D + d] + GSC[2 * D + d] + GSC[3 * D + d] : GSC[63];
}

// ------------------------------------------------------------------------------------------
// Per-chunk packet in the workspace (byte offsets).  Matrices are fp16 64 x 64 with zero upper
// triangles, in the order T, A_qk (, A_kk, A_qu for general gates); tiles are fp16; the gate
// vector is fp32 [512].
//   scalar decay, symmetric gates: matrices, k [64][128], q [64][128] (plain), gates
//     {beta[64], e^{g-gm}[64], e^{gm-g}[64], e^{gm}, e^{gC}, e^{gC-gm}}
//   otherwise: matrices, K+ [64][128], Q+ [64][128], K-^T [128][64] (, U-^T [128][64]),
//     gates {beta[64] (symmetric gates), e^{gm}[128], e^{gC}[128], e^{gC-gm}[128]}
// Every fp16 row is a run of 16-byte units (16 per 128-wide row, 8 per 64-wide row) stored
// XOR-swizzled, unit u of row r at position u ^ swz_key<U>(r), so that the scan can copy a tile
// into LDS as is and still read matrix-core fragments without bank conflicts.
// With FG2's per-channel rate (VP) the packet also carries the scaled values v~ = sqrt(beta) v
// as fp16 [64][128], row-major (the scan copies its value slice from there).
// ------------------------------------------------------------------------------------------
template <bool DCH, bool GEN, bool VP = false>
struct Packet {
  static constexpr bool kScal = !DCH && !GEN;
  static constexpr int nmat = GEN ? 4 : 2;
  static constexpr int mat = 0;
  // bytes per matrix: the six nonzero 16 x 32 blocks of the lower-triangular matrices (tri_pos)
  static constexpr int matb = 6 * 1024;
  static constexpr int kp = mat + nmat * matb;
  static constexpr int qp = kp + C * D * 2;
  static constexpr int kmt = qp + C * D * 2;
  static constexpr int umt = kmt + (kScal ? 0 : D * C * 2);
  static constexpr int gate = umt + (GEN ? D * C * 2 : 0);
  static constexpr int ngate = kScal ? 256 : 512;  // floats
  static constexpr int vt = gate + ngate * 4;
  static constexpr int bytes = vt + (VP ? C * D * 2 : 0);
};

// XOR key of row r in a tile with U 16-byte units per row.  Measured on gfx950 (bank-conflict
// counters over fixed lane patterns), the LDS behaves as follows:
//  - ds_read_b128: 16 lanes of equal lane / 16 per cycle, over 16 slots of 16 bytes, slot
//    ((addr >> 4) ^ (addr >> 10 & 1)) & 15;
//  - ds_read_b64_tr_b16: 32 lanes of equal lane / 32 per cycle, over the 32 8-byte slots of a
//    256-byte window;
//  - ds_write_b64: 16 lanes of equal lane / 16 per cycle, over the 16 8-byte slots of a 128-byte
//    window.
// With these keys a fragment read (rows r0 .. r0 + 15, r0 % 16 == 0) of either tile width and
// the transposing read of a 128-wide tile (rows t0 + 8 g + 0..3, t0 % 32 == 0) are
// conflict-free; fragment-layout writes of 8 bytes per lane into the tiles are 2-way, the least
// that 16 rows at one column allow.  For U = 16 the key / 2 is one-to-one on row bits 0, 1, 3
// (the transposing read), and key ^ (bit 2 of the row, placed at bit 0) on row bits 0..3 (the
// fragment read, after the address hash).
template <int U>
__device__ __forceinline__ int swz_key(int r) {
  if constexpr (U == 16) return ((r >> 3) & 1) | ((r & 3) << 1) | (r & 8);
  else return r & 7;
}

// Half offset of column `col` of row `r` in a swizzled tile with U 16-byte units per row.
template <int U>
__device__ __forceinline__ int swz(int r, int col) {
  return (r * U + ((col >> 3) ^ swz_key<U>(r))) * 8 + (col & 7);
}

// Lower-triangular 64 x 64 fp16 matrices (T, A_qk) of the symmetric-gate packet: only the six
// 16 x 32 blocks (row tile I, column half H) that hold nonzeros are stored, 1 KB each, in the
// order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1); within a block, 16 rows of four 16-byte units with
// unit u of row r at u ^ ((r >> 2) & 3), which makes fragment reads (16 rows at one unit per
// cycle) conflict-free.  The scan keeps all eight blocks in LDS (block 2 I + H), the two upper
// ones zero.
__device__ __forceinline__ int tri_blk(int I, int H) { return I < 2 ? I : 2 * I - 2 + H; }
__device__ __forceinline__ int tri_in(int r, int col) {  // half offset of (r % 16, col % 32) in a block
  return ((r & 15) * 4 + (((col >> 3) & 3) ^ ((r >> 2) & 3))) * 8 + (col & 7);
}
// half offset of element (t, col) in the six-block packet layout (the block must be stored)
__device__ __forceinline__ int tri_pos(int t, int col) { return tri_blk(t >> 4, col >> 5) * 512 + tri_in(t, col); }

// gate-vector slots (floats)
constexpr int GV_BETA = 0;                            // [64]
constexpr int GV_FP = 64, GV_FM = 128, GV_SC = 192;   // scalar decay
constexpr int GV_EM = 64, GV_FC = 192, GV_FCM = 320;  // per-channel decay, [128] each

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// Lane l copies the 16 bytes at its global address `src` to LDS byte `lds_wave` + 16 l
// (`lds_wave` is the same for the whole wave).
__device__ __forceinline__ void dma16(gptr<const char> src, void* lds_wave) {
  __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)lds_wave, 16, 0, 0);
}

// Wait for all of this wave's vector-memory operations (loads, stores, copies to LDS).
__device__ __forceinline__ void vm_wait_all() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt unconstrained
}

// Wait until at most N of this wave's vector-memory operations are outstanding.  Loads complete
// in issue order, so this waits for every load issued before the last N loads.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

// One chunk of prep work: the row of its first token on the token axis ([B * T] for a dense
// batch, the packed axis otherwise), its tokens (1 .. C), its head and its packet index.
struct ChunkRef {
  int64_t tok0;
  int tlen, h;
  int64_t pkt;
};

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

// Per-channel decay or general gates: held to two waves per SIMD (the input prefetch would
// otherwise take the registers of the second resident workgroup).  FG2: the erase array holds
// FG2-GDN's per-channel rate beta ("FG2-GDN ...", section 2, update rule), absorbed here as
// k~ = sqrt(beta) k (every tile and Gram product takes k~) and v~ = sqrt(beta) v (into the
// packet), with the unit gate in place of the per-token erase/write gate.
template <bool DCH, bool GEN, bool FG2 = false>
__global__ __launch_bounds__(kThreads, (DCH || GEN) ? 2 : 1) void chunk_prep_kernel(Problem p, char* __restrict__ ws,
                                                                                     int nchunks, int64_t nblk) {
  static_assert(!(FG2 && GEN), "the per-channel rate keeps the symmetric gates");
  // Packed sequences: the work items are (chunk, head) pairs over the chunk table.
  if (p.chunks) nblk = int64_t(p.H) * *p.nchunks_total;
  using PK = Packet<DCH, GEN, FG2>;
  constexpr int NM = PK::nmat;
  __shared__ __attribute__((aligned(16))) _Float16 KP[C * KS];                 // K+
  __shared__ __attribute__((aligned(16))) _Float16 KM[C * KS];                 // K-
  __shared__ __attribute__((aligned(16))) _Float16 QP[C * KS];                 // Q+
  __shared__ __attribute__((aligned(16))) _Float16 UM[GEN ? C * KS : 8];       // U- (general)
  // fp32 matrix of the solve.  With general gates it takes the place of Q+ (same size), whose
  // last reader runs before it is written: that keeps two workgroups per compute unit.
  __shared__ __attribute__((aligned(16))) float AFA[GEN ? 4 : C * AFS];
  __shared__ __attribute__((aligned(16))) _Float16 TH[C * CS];
  __shared__ float GB[C];
  __shared__ float GSC[4 * D];
  static_assert(C * KS * 2 == C * AFS * 4, "the solve matrix must fit in the Q+ tile");
  float* const AF = GEN ? reinterpret_cast<float*>(QP) : AFA;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  const int d8 = tid & 15, tg = tid >> 4;
  const int T = p.T, H = p.H;
  const gptr<const uint16_t> kin = opaque_gptr(static_cast<const uint16_t*>(p.k));
  const gptr<const uint16_t> qin = opaque_gptr(static_cast<const uint16_t*>(p.q));
  const gptr<const float> ldin = opaque_gptr(p.log_decay);
  const gptr<const float> erin = opaque_gptr(p.erase);
  const bool erase_ch = GEN && p.erase_channel;

  // Inputs of one chunk in registers: thread (token quad tg, channel octet d8) holds tokens
  // 4 tg + r, channels 8 d8 .. + 7; threads < 64 hold token tid's per-head gates.  Tokens past
  // the end load token T - 1 (zeroed where they are used), so every load is unconditional.
  // Per-channel decay with general gates does not prefetch the per-channel erase gates (their
  // registers would spill under the two-workgroup bound); it loads them as the chunk starts,
  // ahead of their first use after the prefix sums.
  constexpr bool kPrefetchErr = GEN && !DCH;
  struct In {
    uint4 kr[4], qr[4];
    float ldr[DCH ? 4 : 1][DCH ? 8 : 1];
    float err[kPrefetchErr ? 4 : 1][kPrefetchErr ? 8 : 1];
    float lds, gb;
  };
  // Work item blk: a dense batch walks (b, h, chunk) with packet index blk; packed sequences
  // walk (chunk, head) over the chunk table.  Work items number fewer than 2^31 (one packet
  // each, and the packets fit in device memory), so the index arithmetic is 32-bit.
  auto chunk_ref = [&](int64_t blk) {
    ChunkRef r;
    const uint32_t ub = uint32_t(blk);
    if (p.chunks) {
      const uint32_t g = ub / uint32_t(H);
      r.h = int(ub - g * uint32_t(H));
      const int4 e = p.chunks[g];
      r.tok0 = e.x;
      r.tlen = e.y;
      r.pkt = int64_t(e.z) + int64_t(r.h) * e.w;
    } else {
      const uint32_t bh = ub / uint32_t(nchunks);
      const int c = int(ub - bh * uint32_t(nchunks));
      const int b = int(bh / uint32_t(H));
      r.h = int(bh) - b * H;
      r.tok0 = int64_t(b) * T + int64_t(c) * C;
      r.tlen = T - c * C < C ? T - c * C : C;
      r.pkt = blk;
    }
    return r;
  };
  auto tok_of = [&](const ChunkRef& cr) {
    return [=](int t) { return (cr.tok0 + (t < cr.tlen ? t : cr.tlen - 1)) * H + cr.h; };
  };
  auto load_err = [&](float (&e)[4][8], const ChunkRef& cr) {
    const auto tok = tok_of(cr);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t base = tok(4 * tg + r) * D + 8 * d8;
      unpack8(gload_f4(erin, base), gload_f4(erin, base + 4), e[r]);
    }
  };
  auto load_in = [&](In& I, int64_t blk) {
    const ChunkRef cr = chunk_ref(blk);
    const auto tok = tok_of(cr);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t base = tok(4 * tg + r) * D + 8 * d8;
      I.kr[r] = gload_u4(kin, base);
      I.qr[r] = gload_u4(qin, base);
      if constexpr (DCH) unpack8(gload_f4(ldin, base), gload_f4(ldin, base + 4), I.ldr[r]);
    }
    if constexpr (kPrefetchErr) {
      if (erase_ch) load_err(I.err, cr);
    }
    if (tid < C) {
      const int64_t ti = tok(tid);
      if constexpr (!DCH) I.lds = ldin[ti];
      if (!erase_ch && !FG2) I.gb = erin[ti];
    }
  };

  // One chunk: prefix sums, operand tiles, gates, Gram matrices, triangular solve.  The solve
  // factor T stays in TH and is written out by the next chunk (or after the last), so that the
  // next chunk's wait for its inputs does not also wait for these stores.
  auto write_t = [&](int64_t pkt) {
    _Float16* wsc = reinterpret_cast<_Float16*>(ws + pkt * PK::bytes + PK::mat);
    const int t = tid >> 2, c0 = (tid & 3) * 16;
    if (c0 < 32 || t >= 32) {  // the blocks that hold nonzeros
      *reinterpret_cast<uint4*>(wsc + tri_pos(t, c0)) = *reinterpret_cast<const uint4*>(TH + t * CS + c0);
      *reinterpret_cast<uint4*>(wsc + tri_pos(t, c0 + 8)) = *reinterpret_cast<const uint4*>(TH + t * CS + c0 + 8);
    }
  };

  // Per-channel decay with general gates or with FG2's rate keeps no chunk in flight (its
  // registers would spill); the second resident workgroup covers its load latency instead.
  constexpr bool kPrefetch = !(DCH && GEN) && !(DCH && FG2);
  In I;
  int64_t blk = blockIdx.x;
  const int64_t gstride = gridDim.x;
  if constexpr (kPrefetch) {
    if (blk < nblk) load_in(I, blk);
  }
  for (int64_t prev = -1; blk < nblk; blk += gstride) {
    const ChunkRef cr = chunk_ref(blk);
    char* pk = ws + cr.pkt * PK::bytes;  // this chunk's packet
    _Float16* wsc = reinterpret_cast<_Float16*>(pk + PK::mat);
    float* gv = reinterpret_cast<float*>(pk + PK::gate);
    if constexpr (!kPrefetch) load_in(I, blk);
    // FG2: this thread's rates and values, issued with the chunk's other inputs
    float rt[FG2 ? 4 : 1][FG2 ? 8 : 1];
    uint4 vr[FG2 ? 4 : 1];
    if constexpr (FG2) {
      const gptr<const uint16_t> vin = opaque_gptr(static_cast<const uint16_t*>(p.v));
      load_err(rt, cr);
      const auto tok = tok_of(cr);
#pragma unroll
      for (int r = 0; r < 4; ++r) vr[r] = gload_u4(vin, tok(4 * tg + r) * D + 8 * d8);
    }
    vm_wait_all();  // this chunk's inputs (loaded one chunk ago) and the older stores

    // ---- inputs, masked past the last token --------------------------------------------
    uint4 kr[4], qr[4];
    float ldr[DCH ? 4 : 1][DCH ? 8 : 1];
    float err[GEN ? 4 : 1][GEN ? 8 : 1];
    float en[GEN && !kPrefetchErr ? 4 : 1][GEN && !kPrefetchErr ? 8 : 1];
    if constexpr (GEN && !kPrefetchErr) {
      if (erase_ch) load_err(en, cr);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = 4 * tg + r < cr.tlen;
      const uint4 z = make_uint4(0, 0, 0, 0);
      kr[r] = ok ? I.kr[r] : z;
      qr[r] = ok ? I.qr[r] : z;
      if constexpr (DCH) {
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) ldr[r][ch] = ok ? I.ldr[r][ch] : 0.f;
      }
      if constexpr (GEN) {
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) err[r][ch] = (ok && erase_ch) ? (kPrefetchErr ? I.err[r][ch] : en[r][ch]) : 0.f;
      }
    }
    // FG2: k~ = sqrt(beta) k replaces k (held as fp16 from here on) and v~ = sqrt(beta) v goes
    // to the packet, right away, so that neither the rates nor the values stay in registers.
    // Rows past the end are zero.
    if constexpr (FG2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = 4 * tg + r < cr.tlen;
        float kf[8], vf[8];
        bf16x8_to_f32(kr[r], kf);
        bf16x8_to_f32(vr[r], vf);
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          const float s = ok ? sqrtf(rt[r][ch]) : 0.f;
          kf[ch] *= s;
          vf[ch] *= s;
        }
        kr[r] = __builtin_bit_cast(uint4, cvt8(kf));
        *reinterpret_cast<half8*>(pk + PK::vt + 2 * ((4 * tg + r) * D + 8 * d8)) = cvt8(vf);
      }
    }
    float lds = 0.f;
    if (tid < C) {
      const bool ok = tid < cr.tlen;
      if constexpr (!DCH) lds = ok ? I.lds : 0.f;
      GB[tid] = (ok && !erase_ch) ? (FG2 ? 1.f : I.gb) : 0.f;
    }

    float g[4][DCH ? 8 : 1];
    chunk_cumsum<DCH>(ldr, lds, g, GSC, tid);

    {
      float gm[8];
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) gm[ch] = chunk_gmid<DCH>(GSC, 8 * d8 + ch);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * tg + r;
        float kf[8], qf[8], kp[8], km[8], qp[8];
        if constexpr (FG2) {  // k~, fp16
          const half8 h = __builtin_bit_cast(half8, kr[r]);
#pragma unroll
          for (int ch = 0; ch < 8; ++ch) kf[ch] = float(h[ch]);
        } else {
          bf16x8_to_f32(kr[r], kf);
        }
        bf16x8_to_f32(qr[r], qf);
        if constexpr (PK::kScal) {
          // scalar decay: plain k and q, in LDS for the Gram products (which take the decay per
          // element, e^{g_t - g_i}) and in the packet for the scan
          const half8 hk = cvt8(kf), hq = cvt8(qf);
          *reinterpret_cast<half8*>(KP + t * KS + 8 * d8) = hk;
          *reinterpret_cast<half8*>(QP + t * KS + 8 * d8) = hq;
          *reinterpret_cast<half8*>(pk + PK::kp + 2 * swz<16>(t, 8 * d8)) = hk;
          *reinterpret_cast<half8*>(pk + PK::qp + 2 * swz<16>(t, 8 * d8)) = hq;
          continue;
        }
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          const float gg = DCH ? g[r][ch] : g[r][0];
          const float fp = clamped_exp(gg - gm[ch]), fm = clamped_exp(gm[ch] - gg);
          kp[ch] = kf[ch] * fp;
          qp[ch] = qf[ch] * fp;
          km[ch] = kf[ch] * fm;
        }
        *reinterpret_cast<half8*>(KP + t * KS + 8 * d8) = cvt8(kp);
        *reinterpret_cast<half8*>(QP + t * KS + 8 * d8) = cvt8(qp);
        *reinterpret_cast<half8*>(KM + t * KS + 8 * d8) = cvt8(km);
        if constexpr (GEN) {
          float um[8];
#pragma unroll
          for (int ch = 0; ch < 8; ++ch) um[ch] = (erase_ch ? err[r][ch] : GB[t]) * km[ch];
          *reinterpret_cast<half8*>(UM + t * KS + 8 * d8) = cvt8(um);
        }
      }
    }

    // per-channel decay: the registers are free, fetch the next chunk's inputs right away
    if constexpr (!PK::kScal && kPrefetch) {
      if (blk + gstride < nblk) load_in(I, blk + gstride);
    }

    // gate vector
    if constexpr (PK::kScal) {
      if (tid < C) {
        const float x = GSC[tid] - GSC[31];
        gv[GV_BETA + tid] = GB[tid];
        gv[GV_FP + tid] = clamped_exp(x);
        gv[GV_FM + tid] = clamped_exp(-x);
      } else if (tid == C) {
        const float gmid = GSC[31], gend = GSC[63];
        *reinterpret_cast<float4*>(gv + GV_SC) =
            make_float4(clamped_exp(gmid), expf(gend), clamped_exp(gend - gmid), 0.f);
      }
    } else {
      if (tid < C) gv[GV_BETA + tid] = GB[tid];
      if (tid < D) {
        const float gmid = chunk_gmid<DCH>(GSC, tid), gend = chunk_gend<DCH>(GSC, tid);
        gv[GV_EM + tid] = clamped_exp(gmid);
        gv[GV_FC + tid] = expf(gend);
        gv[GV_FCM + tid] = clamped_exp(gend - gmid);
      }
    }
    if (prev >= 0) write_t(prev);  // the previous chunk's T, still in TH
    lds_barrier();
    for (int i = tid; i < C * CS; i += kThreads) TH[i] = (_Float16)0.f;

    // Gram tiles, transposed: lane gets A[t = 16 I + l16][i = 16 J + 4 lg + r].
    //   0: A for the solve (symmetric: beta_t A_kk; general: A_ku), strict, fp32 to LDS
    //   1: A_qk (lower), 2: A_kk (strict), 3: A_qu (lower), fp16 to the workspace
    auto gram_tile = [&](int idx) {
      const int which = idx / 10;
      int I0, J0;
      tile_ij(idx - 10 * which, I0, J0);
      const _Float16* Ab = (which == 3 || (GEN && which == 0)) ? UM : PK::kScal ? KP : KM;
      const _Float16* Bb = (which == 1 || which == 3) ? QP : KP;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(frag(Ab, KS, 16 * J0, 32 * ks, lane), frag(Bb, KS, 16 * I0, 32 * ks, lane), acc);
      const int t = 16 * I0 + l16;
      const int i0 = 16 * J0 + 4 * lg;
      if constexpr (PK::kScal) {
        // the decay between token i and token t >= i: e^{g_t - g_i} <= 1 (entries above the
        // diagonal are zeroed below)
        const float gt = GSC[t];
        const float4 gi = *reinterpret_cast<const float4*>(GSC + i0);
        acc[0] *= __expf(fminf(gt - gi.x, 0.f));
        acc[1] *= __expf(fminf(gt - gi.y, 0.f));
        acc[2] *= __expf(fminf(gt - gi.z, 0.f));
        acc[3] *= __expf(fminf(gt - gi.w, 0.f));
      }
      if (which == 0) {
        const float sc = GEN ? 1.f : GB[t];
        float4 v;
        v.x = (i0 + 0 < t) ? sc * acc[0] : 0.f;
        v.y = (i0 + 1 < t) ? sc * acc[1] : 0.f;
        v.z = (i0 + 2 < t) ? sc * acc[2] : 0.f;
        v.w = (i0 + 3 < t) ? sc * acc[3] : 0.f;
        *reinterpret_cast<float4*>(AF + t * AFS + i0) = v;
      } else {
        const bool strict = which == 2;
        half4v hv;
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[r] = (_Float16)((strict ? i0 + r < t : i0 + r <= t) ? acc[r] : 0.f);
        *reinterpret_cast<half4v*>(wsc + which * (PK::matb / 2) + tri_pos(t, i0)) = hv;
      }
    };
    constexpr int NG = 10 * NM;
    // with general gates the solve matrix (tiles 0..9) overwrites Q+ and comes after the rest
    constexpr int G0 = GEN ? 10 : 0;
    // not unrolled with a per-channel decay: unrolled, the fragment loads are
    // hoisted and the registers spill under the two-workgroup bound
    constexpr int kGramUnroll = DCH ? 1 : (NG - G0 + 3) / 4;
#pragma unroll kGramUnroll
    for (int n = 0; n < (NG - G0 + 3) / 4; ++n) {
      const int idx = G0 + wave + 4 * n;
      if (idx < NG) gram_tile(idx);
    }
    // the upper-triangular 16 x 16 tiles (0,1) and (2,3) of the workspace matrices after T share
    // a stored block with nonzeros and are zero (T's come from TH)
    for (int n = wave; n < 2 * (NM - 1); n += 4) {
      const half4v z = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
      const int m = 1 + n / 2, I0 = 2 * (n % 2), J0 = I0 + 1;
      *reinterpret_cast<half4v*>(wsc + m * (PK::matb / 2) + tri_pos(16 * I0 + l16, 16 * J0 + 4 * lg)) = z;
    }
    // operand tiles for the scan (per-channel decay or general gates): K+, Q+ row-major;
    // K-, U- transposed ([channel][token]); all swizzled
    if constexpr (!PK::kScal) {
#pragma unroll
      for (int i = 0; i < C * D / 8 / kThreads; ++i) {
        const int u = tid + kThreads * i;
        const int t = u >> 4, c8 = ((u & 15) ^ swz_key<16>(t)) * 8;  // stored unit u & 15 holds column c8
        *reinterpret_cast<uint4*>(pk + PK::kp + 16 * u) = *reinterpret_cast<const uint4*>(KP + t * KS + c8);
        *reinterpret_cast<uint4*>(pk + PK::qp + 16 * u) = *reinterpret_cast<const uint4*>(QP + t * KS + c8);
      }
#pragma unroll
      for (int i = 0; i < C * D / 8 / kThreads; ++i) {
        const int d = tid & (D - 1), t0 = 8 * ((tid >> 7) + 2 * i);
        half8 x;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = KM[(t0 + j) * KS + d];
        *reinterpret_cast<half8*>(pk + PK::kmt + 2 * swz<8>(d, t0)) = x;
        if constexpr (GEN) {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = UM[(t0 + j) * KS + d];
          *reinterpret_cast<half8*>(pk + PK::umt + 2 * swz<8>(d, t0)) = x;
        }
      }
    }
    lds_barrier();
    if constexpr (GEN) {
      // A_ku into the solve matrix, now that Q+ has been read for the last time
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        const int idx = wave + 4 * n;
        if (idx < 10) gram_tile(idx);
      }
      lds_barrier();
    }
    // scalar decay: fetch the next chunk's inputs only now, in flight during the solve, which
    // keeps them out of the Gram stage's registers (measured faster for this variant)
    if constexpr (PK::kScal) {
      if (blk + gstride < nblk) load_in(I, blk + gstride);
    }

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
    if (blk + gstride >= nblk) write_t(cr.pkt);  // this workgroup's last chunk
    prev = cr.pkt;
  }
}

// ------------------------------------------------------------------------------------------
// Scan: the chunks of one (b, h, value slice) in order, eight waves per workgroup.
// ------------------------------------------------------------------------------------------
constexpr int kScanWaves = 8;
constexpr int kScanThreads = 64 * kScanWaves;

// Fragment (as frag()) of a swizzled tile with U 16-byte units per row.
template <int U>
__device__ __forceinline__ half8 frag_s(const _Float16* base, int row0, int k0, int lane) {
  return *reinterpret_cast<const half8*>(base + swz<U>(row0 + (lane & 15), k0 + 8 * (lane >> 4)));
}

// Fragment (as frag()) of rows 16 I .. + 15, columns 32 H .. + 31 of a lower-triangular matrix
// held in LDS as eight 16 x 32 blocks (block 2 I + H, layout as tri_in).
__device__ __forceinline__ half8 frag_tri(const _Float16* base, int I, int H, int lane) {
  return *reinterpret_cast<const half8*>(base + (2 * I + H) * 512 + tri_in(lane & 15, 8 * (lane >> 4)));
}

// LDS layout of the register-staged scan (general gates).
template <bool GEN, bool SCAL, int DVS>
struct ScanLayout {
  static_assert(GEN && !SCAL, "the register-staged scan serves general gates");
  // Every tile in the packet's layout (swizzled, see swz_key; the matrices as 16 x 32 blocks, see
  // tri_pos), so units copy straight across and fragment reads are conflict-free.
  static constexpr int kp = 0;                 // K+       [64][128] half
  static constexpr int qp = kp + C * D * 2;    // Q+       [64][128]
  static constexpr int kmt = qp + C * D * 2;   // K-^T     [128][64]
  static constexpr int umt = kmt + D * C * 2;  // U-^T     [128][64]
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
template <bool DCH, bool GEN, bool WCH, int DVS>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(Problem p, const char* __restrict__ ws) {
  static_assert(GEN, "symmetric gates use chunk_scan_sym_kernel");
  using PK = Packet<DCH, GEN>;
  using L = ScanLayout<GEN, false, DVS>;
  constexpr int NM = PK::nmat;
  constexpr int NCT = DVS / 16;   // 16-column tiles of the value slice
  constexpr int VPT = DVS / 8;    // value columns per thread in the V load
  constexpr int NTU = 8;  // 16-byte operand-tile units per thread (K+, Q+, K-^T, U-^T)
  constexpr int PF = 1;   // chunks of prefetch in flight
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
    uint4 tl[NTU];            // K+, Q+, K-^T, U-^T units
    float4 sc[3];             // per-channel e^{gm}, e^{gC}, e^{gC-gm} of this thread's 4 rows
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
    // S~^T = (Diag(e^{gm}) S)^T; the end-of-chunk factors of this wave's rows stay in registers.
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
        ak[ks] = frag_s<8>(KMT, 16 * wave, 32 * ks, lane);
        au[ks] = frag_s<8>(UMT, 16 * wave, 32 * ks, lane);
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
  Pref PA;
  load(PA, 0);
  int c = 0;
  for (; c < nfull; ++c) step(Flag<false>(), c, PA);
  if (c < nchunks) step(Flag<true>(), c, PA);

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
// gfx950 transposing LDS read (ds_read_b64_tr_b16): lane 16 g + 4 a + b receives as element j
// (0..3) the 16-bit element b of the 8 bytes at the address that lane 16 g + a + 4 j supplies.
typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4 lds_half4;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
__device__ __forceinline__ half4v ld_tr16(const _Float16* p) {
  return __builtin_bit_cast(half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_half4*)p));
}
__device__ __forceinline__ short4v ld_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
}

// frag_s of the transposed tile: A[row = d][k = t] = base[t][d] (base swizzled, 16 units per
// row).  Lane 16 g + m supplies row t0 + 8 g + m / 4 (and 4 rows on), columns d0 + 4 (m % 4)
// .. + 3, so lane 16 g + l16 receives base[t0 + 8 g + 0..7][d0 + l16].
__device__ __forceinline__ half8 frag_ts(const _Float16* base, int d0, int t0, int lane) {
  const int m = lane & 15;
  const int t = t0 + 8 * (lane >> 4) + (m >> 2), d = d0 + 4 * (m & 3);
  const half4v lo = ld_tr16(base + swz<16>(t, d));
  const half4v hi = ld_tr16(base + swz<16>(t + 4, d));
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// FG2: the values are FG2's v~ = sqrt(beta) v, fp16 in the packet, instead of the bf16 input.
template <bool DCH, int DVS, bool FG2 = false>
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
  // (eight 16 x 32 blocks each, see tri_pos); batch 3: K-^T [128][64] (per-channel decay).
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
  __shared__ __attribute__((aligned(16))) _Float16 DT2[SCAL ? DVS * C : 8];  // (Diag(e^{gm-g}) delta)^T

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
  // the start of the chunk; (2) T and A_qk, read from the D stage on; (3) K-^T (per-channel
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
    // S~^T = (Diag(e^{gm}) S)^T
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
    fetch2(Y, cn);

    // ---- D: delta = T R, stored transposed ---------------------------------------------
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
      if constexpr (SCAL) {
        // K-^T delta = k^T (Diag(e^{gm - g}) delta): the state update takes the scaled copy
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
        ak[ks] = SCAL ? frag_ts(X.kp, 16 * wave, 32 * ks, lane) : frag_s<8>(X.km, 16 * wave, 32 * ks, lane);
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

template <bool DCH, int DVS, bool FG2>
hipError_t launch_scan_sym(const Problem& p, const char* ws, hipStream_t stream) {
  dim3 grid(unsigned(p.B * p.H), unsigned(D / DVS));
  hipLaunchKernelGGL((chunk_scan_sym_kernel<DCH, DVS, FG2>), grid, dim3(kScanThreads), 0, stream, p, ws);
  return hipGetLastError();
}

template <bool DCH, int DVS>
hipError_t launch_scan_gen(const Problem& p, const char* ws, hipStream_t stream) {
  dim3 grid(unsigned(p.B * p.H), unsigned(D / DVS));
  if (p.write_channel)
    hipLaunchKernelGGL((chunk_scan_kernel<DCH, true, true, DVS>), grid, dim3(kScanThreads), 0, stream, p, ws);
  else
    hipLaunchKernelGGL((chunk_scan_kernel<DCH, true, false, DVS>), grid, dim3(kScanThreads), 0, stream, p, ws);
  return hipGetLastError();
}

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
  hipLaunchKernelGGL((chunk_prep_kernel<DCH, GEN, FG2>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p, ws, nchunks,
                     nblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Fill the 256 compute units with (b, h, value-slice) workgroups while keeping the slices
  // (each stages its chunk's operand tiles) as wide as that allows.
  const int64_t bh = int64_t(p.B) * p.H;
  if constexpr (GEN) {
    return bh >= 64 ? launch_scan_gen<DCH, 32>(p, ws, stream) : launch_scan_gen<DCH, 16>(p, ws, stream);
  } else {
    return bh >= 64 ? launch_scan_sym<DCH, 32, FG2>(p, ws, stream) : launch_scan_sym<DCH, 16, FG2>(p, ws, stream);
  }
}

int64_t packet_bytes(bool symmetric, bool decay_channel, bool rate_sqrt) {
  if (rate_sqrt) return decay_channel ? Packet<true, false, true>::bytes : Packet<false, false, true>::bytes;
  return !symmetric ? Packet<true, true>::bytes : decay_channel ? Packet<true, false>::bytes : Packet<false, false>::bytes;
}

int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }

}  // namespace

size_t chunk128_workspace_bytes(int B, int T, int H, bool symmetric, bool decay_channel, bool rate_sqrt) {
  const int64_t nchunks = (int64_t(T) + C - 1) / C;
  return size_t(int64_t(B) * H * nchunks * packet_bytes(symmetric, decay_channel, rate_sqrt));
}

// Packed sequences: packets of at most varlen_max_chunks chunks per head, then the chunk
// table, the sequence table, the sequence order and the chunk count.
size_t chunk128_varlen_workspace_bytes(int nseq, int T, int H, bool symmetric, bool decay_channel, bool rate_sqrt) {
  const int64_t maxc = varlen_max_chunks(nseq, T);
  return size_t(int64_t(H) * maxc * packet_bytes(symmetric, decay_channel, rate_sqrt) + round256(maxc * 16) +
                round256(int64_t(nseq) * 16) + round256(int64_t(nseq) * 4) + 256);
}

hipError_t launch_chunk128_varlen(Problem p, const int* cu, void* workspace, hipStream_t stream) {
  const int64_t maxc = varlen_max_chunks(p.B, p.T);
  char* ws = static_cast<char*>(workspace);
  char* tables = ws + int64_t(p.H) * maxc * packet_bytes(p.symmetric, p.decay_channel, p.rate_sqrt);
  int4* chunks = reinterpret_cast<int4*>(tables);
  int4* seqs = reinterpret_cast<int4*>(tables + round256(maxc * 16));
  int* order = reinterpret_cast<int*>(tables + round256(maxc * 16) + round256(int64_t(p.B) * 16));
  int* total = order + round256(int64_t(p.B) * 4) / 4;
  hipError_t e = launch_varlen_setup(cu, p.B, p.T, p.H, C, seqs, chunks, total, order, stream);
  if (e != hipSuccess) return e;
  p.seqs = seqs;
  p.chunks = chunks;
  p.nchunks_total = total;
  p.order = order;
  return launch_chunk128(p, workspace, stream);
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
