// Layouts and fragment helpers shared by the matrix-core chunk kernels (forward prep and
// scans, adjoint scan, chunk gradients): the per-chunk packet, the swizzled fp16 tiles and
// triangular blocks it holds, and the LDS reads that feed v_mfma_f32_16x16x{16,32}_f16.
#pragma once

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

__device__ __forceinline__ half4v cvt4(f32x4 a) {
  half4v h;
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = (_Float16)a[r];
  return h;
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 u, float* f) {
  f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
  f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
  f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}

// v when ok, else zero
__device__ __forceinline__ uint4 mask4(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

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

// The 4 x 4 transpose within each quad of lanes: lane b of a quad holds x = row b of a 4 x 4
// block (x[r] = A[b][r]) and receives column b (A[r][b]).  Two DPP exchanges: the off-diagonal
// 2 x 2 blocks between lanes 2 apart, then the off-diagonal elements of each 2 x 2 block between
// neighbouring lanes.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x) {
  const int b = threadIdx.x & 3;
  auto xchg = [](float v, int ctrl) {  // v of the quad partner that ctrl names
    return ctrl == 0x4e ? __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, false))
                        : __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false));
  };
  const bool hi2 = (b & 2) != 0, odd = (b & 1) != 0;
  // lanes 0, 1 send elements 2, 3 and take the partner's 0, 1 there; lanes 2, 3 the other way
  const float s0 = xchg(hi2 ? x[0] : x[2], 0x4e), s1 = xchg(hi2 ? x[1] : x[3], 0x4e);
  f32x4 y = x;
  if (hi2) { y[0] = s0; y[1] = s1; } else { y[2] = s0; y[3] = s1; }
  // even lanes send elements 1, 3 and take the partner's 0, 2 there; odd lanes the other way
  const float t0 = xchg(odd ? y[0] : y[1], 0xb1), t1 = xchg(odd ? y[2] : y[3], 0xb1);
  f32x4 z = y;
  if (odd) { z[0] = t0; z[2] = t1; } else { z[1] = t0; z[3] = t1; }
  return z;
}

// ------------------------------------------------------------------------------------------
// Per-chunk packet in the workspace (byte offsets).  Matrices are fp16 64 x 64 with zero upper
// triangles, in the order T, A_qk (, A_kk, A_qu for general gates); tiles are fp16; the gate
// vector is fp32 [512].
//   scalar decay, symmetric gates: matrices, k [64][128], q [64][128] (plain), gates
//     {beta[64], e^{g}[64], e^{g_C - g}[64], 1, e^{g_C}, 1}
//   otherwise: matrices, K+ [64][128], Q+ [64][128], K^end [64][128] (, U^end [64][128]), gates
//     {beta[64] (symmetric gates), 1[128], e^{g_C}[128], 1[128]}
// Every fp16 row is a run of 16-byte units (16 per 128-wide row) stored XOR-swizzled, unit u of
// row r at position u ^ swz_key<16>(r), so that the scan can copy a tile into LDS as is and
// still read matrix-core fragments (and, from K^end, transposed fragments) without bank
// conflicts.  With FG2's per-channel rate (VP) the packet also carries the scaled values
// v~ = sqrt(beta) v as fp16 [64][128], row-major (the scan copies its value slice from there).
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

// Fragment (as frag()) of a swizzled tile with U 16-byte units per row.
template <int U>
__device__ __forceinline__ half8 frag_s(const _Float16* base, int row0, int k0, int lane) {
  return *reinterpret_cast<const half8*>(base + swz<U>(row0 + (lane & 15), k0 + 8 * (lane >> 4)));
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


// Fragment (as frag()) of rows 16 I .. + 15, columns 32 H .. + 31 of a lower-triangular matrix
// held in LDS as eight 16 x 32 blocks (block 2 I + H, layout as tri_in).
__device__ __forceinline__ half8 frag_tri(const _Float16* base, int I, int H, int lane) {
  return *reinterpret_cast<const half8*>(base + (2 * I + H) * 512 + tri_in(lane & 15, 8 * (lane >> 4)));
}

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


// frag_ts of a lower-triangular matrix held in LDS as eight 16 x 32 blocks (block 2 I + H, layout
// as tri_in): lane 16 g + l16 receives A[r0 + 8 g + 0..7][c0 + l16] (c0 % 16 == 0, r0 % 8 == 0).
__device__ __forceinline__ half8 frag_tri_t(const _Float16* base, int c0, int r0, int lane) {
  const int m = lane & 15;
  const int r = r0 + 8 * (lane >> 4) + (m >> 2), c = c0 + 4 * (m & 3);
  const half4v lo = ld_tr16(base + (2 * (r >> 4) + (c >> 5)) * 512 + tri_in(r, c));
  const half4v hi = ld_tr16(base + (2 * ((r + 4) >> 4) + (c >> 5)) * 512 + tri_in(r + 4, c));
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}


// One chunk of prep work: the row of its first token on the token axis ([B * T] for a dense
// batch, the packed axis otherwise), its tokens (1 .. C), its head and its packet index.
struct ChunkRef {
  int64_t tok0;
  int tlen, h;
  int64_t pkt;
};

// One chunk of prep work, from its work-item index: a dense batch walks (b, h, chunk) with
// packet index blk; packed sequences walk (chunk, head) over the chunk table.  Work items number
// fewer than 2^31 (one packet each, and the packets fit in device memory), so the index
// arithmetic is 32-bit.
__device__ __forceinline__ ChunkRef chunk_ref_of(const Problem& p, int64_t blk, int nchunks) {
  ChunkRef r;
  const uint32_t ub = uint32_t(blk);
  if (p.chunks) {
    const uint32_t g = ub / uint32_t(p.H);
    r.h = int(ub - g * uint32_t(p.H));
    const int4 e = p.chunks[g];
    r.tok0 = e.x;
    r.tlen = e.y;
    r.pkt = int64_t(e.z) + int64_t(r.h) * e.w;
  } else {
    const uint32_t bh = ub / uint32_t(nchunks);
    const int c = int(ub - bh * uint32_t(nchunks));
    const int b = int(bh / uint32_t(p.H));
    r.h = int(bh) - b * p.H;
    r.tok0 = int64_t(b) * p.T + int64_t(c) * C;
    r.tlen = p.T - c * C < C ? p.T - c * C : C;
    r.pkt = blk;
  }
  return r;
}

}  // namespace
}  // namespace dr
