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
// Kernel 1, one wave per (b, h, group of 256 / dk value columns): lane = column x row group,
// four rows of one column per lane:
//   pass 1 runs the forward and stores the state at the start of every 64-token chunk;
//   pass 2 takes the chunks backwards: it recomputes the chunk's states from its checkpoint
//   into a scratch area of its own, then walks the chunk's tokens backwards through the adjoint
//   above.  Column sums (m, dm, dv~) are lane sums plus cross-lane steps; row sums (the per-row
//   parts of dq, du, dk and d(log a), summed over this wave's columns) are reduced over the
//   column lanes and stored per column group.
// The column groups of 32 value columns of one (b, h) share a workgroup and sum their row parts
// in LDS before storing them, so one row part per workgroup reaches memory.
// Kernel 2 sums the workgroups' row parts, applies the per-row factors (e, k, a) and forms
// the gate gradients (summed over channels for a per-head gate; the erase and write parts added
// for a shared gate).
// Every state value is read and written by the lane that owns it; the only barrier is the one
// per token before the LDS sum.  The two kernels are ordered by the stream.

#include "dr_device.h"
#include "dr_internal.h"

namespace dr {
namespace {

constexpr int CK = 64;  // tokens per checkpoint

// Value columns per wave: the fewest that leave a lane four rows (dk * cols / 64 == 4): more,
// narrower waves run side by side on a SIMD.
__host__ __device__ constexpr int cols_for(int dk) { return 256 / dk; }

// x of the lane that the DPP control CTRL selects within this lane's row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the lanes of one column (lanes c + COLS i), in every one of them: within a row of 16
// lanes, rotations by 4 (4 columns) and by 8 add the lanes of the same column; then the gfx950
// row swaps: swapping rows
// 1 <-> 0 and 3 <-> 2 of a value with itself and adding both results gives each lane the sum of
// its pair of rows, and the half-wave swap adds the other pair.  Paired lanes add in the same
// order, so every lane of the column holds the same sum.
template <int COLS>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (COLS == 2) x += dpp<0x122>(x);  // row rotate by 2: lanes 2 apart
  if constexpr (COLS <= 4) x += dpp<0x124>(x);  // row rotate by 4: lanes 4 apart
  if constexpr (COLS <= 8) x += dpp<0x128>(x);  // row rotate by 8: the other half-row
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reduce-scatter of N values per lane over the COLS lanes of a row group: DPP pairings (row
// mirror for 16 columns, then half-row mirror, quad swaps 2 and 1 apart); at each one a lane
// keeps the half of its values that its lane bit selects, adds the partner's copy of that half,
// and sends the other half.  Afterwards lane c holds the full sums of rows rs_row(c) .. +
// rs_count - 1 in v[0 ..]; when fewer values than lanes remain, a pairing finds a single value
// and just adds the partner's, so several lanes hold the same rows (rs_owner marks one).
template <int CTRL, int BIT, int N>
__device__ __forceinline__ void rs_stage(float* v, int c) {
  if constexpr (N > 1) {
    constexpr int H = N / 2;
    const bool low = ((c >> BIT) & 1) == 0;
#pragma unroll
    for (int m = 0; m < H; ++m) {
      const float keep = low ? v[m] : v[m + H];
      const float send = low ? v[m + H] : v[m];
      v[m] = keep + dpp<CTRL>(send);
    }
  } else {
    v[0] += dpp<CTRL>(v[0]);
  }
}
template <int COLS, int N>
__device__ __forceinline__ void row_scatter_sum(float* v, int c) {
  if constexpr (COLS == 16) {
    rs_stage<0x140, 3, N>(v, c);
    rs_stage<0x141, 2, (N > 1 ? N / 2 : 1)>(v, c);
    rs_stage<0x4E, 1, (N > 2 ? N / 4 : 1)>(v, c);
    rs_stage<0xB1, 0, (N > 4 ? N / 8 : 1)>(v, c);
  } else if constexpr (COLS == 8) {
    rs_stage<0x141, 2, N>(v, c);
    rs_stage<0x4E, 1, (N > 1 ? N / 2 : 1)>(v, c);
    rs_stage<0xB1, 0, (N > 2 ? N / 4 : 1)>(v, c);
  } else if constexpr (COLS == 4) {
    rs_stage<0x4E, 1, N>(v, c);
    rs_stage<0xB1, 0, (N > 1 ? N / 2 : 1)>(v, c);
  } else {
    rs_stage<0xB1, 0, N>(v, c);
  }
}
template <int COLS, int N>
__device__ __forceinline__ int rs_row(int c) {
  if constexpr (COLS == 16)
    return (N > 1 ? (N / 2) * ((c >> 3) & 1) : 0) + (N > 2 ? (N / 4) * ((c >> 2) & 1) : 0) +
           (N > 4 ? (N / 8) * ((c >> 1) & 1) : 0) + (N > 8 ? (N / 16) * (c & 1) : 0);
  else if constexpr (COLS == 8)
    return (N > 1 ? (N / 2) * ((c >> 2) & 1) : 0) + (N > 2 ? (N / 4) * ((c >> 1) & 1) : 0) +
           (N > 4 ? (N / 8) * (c & 1) : 0);
  else if constexpr (COLS == 4)
    return (N > 1 ? (N / 2) * ((c >> 1) & 1) : 0) + (N > 2 ? (N / 4) * (c & 1) : 0);
  else
    return N > 1 ? (N / 2) * (c & 1) : 0;
}
template <int COLS, int N>
constexpr int rs_count = N >= COLS ? N / COLS : 1;
template <int COLS, int N>
__device__ __forceinline__ bool rs_owner(int c) {
  if constexpr (COLS == 16)
    return (N > 8 || (c & 1) == 0) && (N > 4 || (c & 2) == 0) && (N > 2 || (c & 4) == 0) && (N > 1 || (c & 8) == 0);
  else if constexpr (COLS == 8)
    return (N > 4 || (c & 1) == 0) && (N > 2 || (c & 2) == 0) && (N > 1 || (c & 4) == 0);
  else if constexpr (COLS == 4)
    return (N > 2 || (c & 1) == 0) && (N > 1 || (c & 2) == 0);
  else
    return N > 1 || (c & 1) == 0;
}

// Workspace layout of the backward (offsets in floats).  Packed sequences (p.B of them over p.T
// tokens, one token row each): the checkpoints of sequence n, head h and column group s start at
// chunk nslice * H * (chunks before n) + (h * nslice + s) * (chunks of n), at most
// nslice * H * varlen_max_chunks chunks in all.
struct BwdLayout {
  int64_t nslice, nck, bth;
  int wpg;          // column groups (waves) per workgroup: their row parts are summed in LDS
  int64_t ngroups;  // workgroups per (b, h): one stored row part each
  int64_t ckpt, states, parts, tmp_dw, total;
  __host__ __device__ BwdLayout(const Problem& p, bool packed) {
    const int cols = cols_for(p.dk);
    nslice = p.dv / cols;
    // waves per workgroup: 32 value columns (at most 16 waves), so a workgroup stores one row
    // part per 32 columns whatever the wave width
    wpg = int(32 / cols) < nslice ? int(32 / cols) : int(nslice);
    ngroups = nslice / wpg;
    nck = (int64_t(p.T) + CK - 1) / CK;
    bth = packed ? int64_t(p.T) * p.H : int64_t(p.B) * p.T * p.H;
    const int64_t waves = int64_t(p.B) * p.H * nslice;
    const int64_t nckpt = packed ? nslice * p.H * varlen_max_chunks(p.B, p.T) : waves * nck;
    ckpt = 0;                                             // [nckpt][dk][cols]
    states = ckpt + nckpt * p.dk * cols;                  // [waves][CK][dk][cols]
    parts = states + waves * CK * p.dk * cols;            // [4][ngroups][bth][dk]
    tmp_dw = parts + 4 * ngroups * bth * p.dk;            // [bth][dv]: v * dv~
    total = tmp_dw + bth * p.dv;
  }
};

template <int DK>
__global__ __launch_bounds__(1024) void bwd_token_kernel(Problem p, BwdArgs g, float* __restrict__ ws) {
  constexpr int kCols = cols_for(DK);
  constexpr int RPL = DK * kCols / 64;  // rows per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & (kCols - 1);
  const int grp = lane / kCols;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh - b * p.H;
  const int dv = p.dv;
  const int nw = blockDim.x >> 6;  // column groups in this workgroup
  const int slice = blockIdx.y * nw + wave;
  const int j = slice * kCols + c;
  const int row0 = grp * RPL;
  const bool bf = p.qkv_bf16;
  const BwdLayout L(p, p.seqs != nullptr);
  const int64_t wave_id = int64_t(bh) * L.nslice + slice;
  // this wave's sequence: a dense batch row, or a packed sequence from the table
  int64_t tok_base = int64_t(b) * p.T;
  int T = p.T;
  int64_t nck = L.nck;
  float* ck = ws + L.ckpt + wave_id * L.nck * DK * kCols;
  if (p.seqs) {
    const int4 e = p.seqs[b];  // {first token, tokens, H * chunks before, chunks}
    tok_base = e.x;
    T = e.y;
    nck = e.w;
    ck = ws + L.ckpt + (L.nslice * e.z + int64_t(h * L.nslice + slice) * e.w) * DK * kCols;
  }
  float* st = ws + L.states + wave_id * CK * DK * kCols;
  // A state slice in the scratch area is stored lane-major (lane l's RPL values contiguous), so
  // that a lane saves or restores its part with RPL / 4 16-byte accesses.
  auto save = [&](float* dst, const float (&v)[RPL]) {
#pragma unroll
    for (int i = 0; i < RPL; i += 4)
      *reinterpret_cast<f32x4*>(dst + lane * RPL + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
  };
  auto restore = [&](const float* src, float (&v)[RPL]) {
#pragma unroll
    for (int i = 0; i < RPL; i += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + lane * RPL + i);
      v[i] = x[0];
      v[i + 1] = x[1];
      v[i + 2] = x[2];
      v[i + 3] = x[3];
    }
  };

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
    if (p.rate_sqrt) {  // FG2's rate: the scaled key sqrt(beta) k with a unit erase, v~ = sqrt(beta) v
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        x.k[r] *= sqrtf(x.e[r]);
        x.e[r] = 1.f;
      }
      x.w = sqrtf(x.w);
    }
  };
  // one forward token: s <- S_t from s = S_{t-1}
  auto step = [&](float (&s)[RPL], const Tok& x) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      s[r] *= x.a[r];
      m = fmaf(x.k[r], s[r], m);
    }
    m = group_sum<kCols>(m);
    const float wv = x.w * x.v;
#pragma unroll
    for (int r = 0; r < RPL; ++r) s[r] = fmaf(-x.e[r] * x.k[r], m, fmaf(x.k[r], wv, s[r]));
  };
  auto token = [&](int t) { return (tok_base + t) * p.H + h; };

  // ---- pass 1: forward, checkpoint every CK tokens -------------------------------------------
  float s[RPL];
  const int64_t sbase = int64_t(bh) * DK * dv + j;
#pragma unroll
  for (int r = 0; r < RPL; ++r) s[r] = p.S0 ? p.S0[sbase + int64_t(row0 + r) * dv] : 0.f;
  // Every loop loads the next token's inputs before working on the current one, so that one
  // token's computation covers the next one's load latency.
  Tok x, nx;
  if (T > 0) load_tok(nx, token(0));
  for (int t = 0; t < T; ++t) {
    x = nx;
    if (t + 1 < T) load_tok(nx, token(t + 1));
    if (t % CK == 0) {
      save(ck + int64_t(t / CK) * DK * kCols, s);
    }
    step(s, x);
  }

  // ---- pass 2: the adjoint, chunk by chunk from the last ----------------------------------------
  float G[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) G[r] = g.dS_T ? g.dS_T[sbase + int64_t(row0 + r) * dv] : 0.f;
  float* parts = ws + L.parts;
  const int64_t pstride = L.ngroups * L.bth * DK;  // between the four row-part arrays
  // the workgroup's column groups' row parts of one token, alternating between two buffers
  __shared__ float red[2][16][4][DK];
  for (int64_t ci = nck - 1; ci >= 0; --ci) {
    const int t0 = int(ci * CK), t1 = t0 + CK < T ? t0 + CK : T;
    restore(ck + ci * DK * kCols, s);
    load_tok(nx, token(t0));
    for (int t = t0; t < t1; ++t) {  // S_{t-1} of every token of the chunk
      x = nx;
      if (t + 1 < t1) load_tok(nx, token(t + 1));
      save(st + int64_t(t - t0) * DK * kCols, s);
      step(s, x);
    }
    // the adjoint walk: token t's inputs, q, dO and S_{t-1}, loaded one token ahead
    float nq[RPL], nsp[RPL], ndO;
    auto load_back = [&](int t) {
      const int64_t tok = token(t);
      load_tok(nx, tok);
      load_rows<RPL>(p.q, tok * DK + row0, bf, nq);
      restore(st + int64_t(t - t0) * DK * kCols, nsp);
      ndO = g.dO[tok * dv + j];
    };
    load_back(t1 - 1);
    for (int t = t1 - 1; t >= t0; --t) {
      const int64_t tok = token(t);
      float qr[RPL], sp[RPL];
      x = nx;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        qr[r] = nq[r];
        sp[r] = nsp[r];
      }
      const float dO = ndO;
      if (t > t0) load_back(t - 1);
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) m = fmaf(x.k[r], x.a[r] * sp[r], m);
      m = group_sum<kCols>(m);
      const float vw = x.w * x.v;
      // row parts, summed over this wave's columns (reduce-scatter: lane c holds rows
      // rs_row(c) ..), then over the workgroup's column groups through LDS
      const int buf = t & 1;
      const int prow = row0 + rs_row<kCols, RPL>(c);
      const bool owner = rs_owner<kCols, RPL>(c);
      auto put = [&](float* part, int which) {
        row_scatter_sum<kCols, RPL>(part, c);
        if (owner) {
#pragma unroll
          for (int i = 0; i < rs_count<kCols, RPL>; ++i) red[buf][wave][which][prow + i] = part[i];
        }
      };
      float dm = 0.f, dvw = 0.f;
      float pa[RPL], pb[RPL];
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const float Sp = x.a[r] * sp[r];
        const float St = fmaf(-x.e[r] * x.k[r], m, fmaf(x.k[r], vw, Sp));
        G[r] = fmaf(qr[r], dO, G[r]);
        pa[r] = St * dO;    // dq
        pb[r] = -G[r] * m;  // du
        dm = fmaf(-G[r] * x.e[r], x.k[r], dm);
        dvw = fmaf(G[r], x.k[r], dvw);
      }
      put(pa, 0);
      put(pb, 1);
      dm = group_sum<kCols>(dm);
      dvw = group_sum<kCols>(dvw);
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const float Sp = x.a[r] * sp[r];
        pa[r] = fmaf(G[r], vw, Sp * dm);  // dk, less the erase part
        const float Gp = fmaf(x.k[r], dm, G[r]);
        pb[r] = Gp * sp[r];  // d(log a) / a
        G[r] = x.a[r] * Gp;
      }
      put(pa, 2);
      put(pb, 3);
      // Every wave of the workgroup walks the same tokens, so all meet here; a buffer is written
      // again two tokens later, after the next token's barrier, which every reader has passed.
      lds_barrier();
      for (int i = threadIdx.x; i < 4 * DK; i += blockDim.x) {
        const int which = i / DK, row = i - which * DK;
        float sum = 0.f;
        for (int w = 0; w < nw; ++w) sum += red[buf][w][which][row];
        parts[which * pstride + (int64_t(blockIdx.y) * L.bth + tok) * DK + row] = sum;
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
// parts: [4][ngroups][bth][dk] row parts; tmp_dw: [bth][dv] v * dv~.
__global__ __launch_bounds__(128) void bwd_reduce_kernel(Problem p, BwdArgs g, const float* __restrict__ parts,
                                                         const float* __restrict__ tmp_dw, int64_t ngroups,
                                                         int64_t bth) {
  __shared__ float red[2];
  const int64_t tok = blockIdx.x;
  const int i = threadIdx.x;
  const int dk = p.dk, dv = p.dv;
  const int64_t pstride = ngroups * bth * dk;
  float sq = 0.f, sdu = 0.f, skw = 0.f, sda = 0.f;
  float de = 0.f, dla = 0.f, dwv = 0.f;
  if (i < dk) {
    for (int64_t s = 0; s < ngroups; ++s) {
      const float* pb = parts + (s * bth + tok) * dk + i;
      sq += pb[0];
      sdu += pb[pstride];
      skw += pb[2 * pstride];
      sda += pb[3 * pstride];
    }
    const float k = load_qkv(p.k, tok * dk + i, p.qkv_bf16);
    const float e = p.erase_channel ? p.erase[tok * dk + i] : p.erase[tok];
    const float a = expf(p.decay_channel ? p.log_decay[tok * dk + i] : p.log_decay[tok]);
    g.dq[tok * dk + i] = sq;
    dla = a * sda;
    if (p.rate_sqrt) {
      // FG2's rate: the parts are for the scaled key k~ = sqrt(beta) k with a unit erase, so
      // dk~ = skw + sdu; dk = sqrt(beta) dk~, and beta's gradient gathers k dk~ and (below)
      // v dv~, each over 2 sqrt(beta)
      const float rt = sqrtf(e), dkt = skw + sdu;
      g.dk[tok * dk + i] = rt * dkt;
      de = k * dkt / (2.f * rt);
    } else {
      g.dk[tok * dk + i] = fmaf(e, sdu, skw);
      de = k * sdu;
    }
  }
  if (i < dv) {
    dwv = tmp_dw[tok * dv + i];
    if (p.rate_sqrt) dwv /= 2.f * sqrtf(p.erase[tok * dk + i]);  // v dv~ / (2 sqrt(beta)); dk == dv
  }
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

size_t bwd_workspace_bytes(const Problem& p) { return size_t(BwdLayout(p, false).total) * 4; }

// Packed sequences: the sequence table and the chunk count first, then the layout above.
static int64_t bwd_tables_bytes(int nseq) { return (int64_t(nseq) * 16 + 255) / 256 * 256 + 256; }

size_t bwd_varlen_workspace_bytes(const Problem& p) {
  return size_t(bwd_tables_bytes(p.B) + BwdLayout(p, true).total * 4);
}

hipError_t launch_bwd_varlen(Problem p, const int* cu, const BwdArgs& g, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  int4* seqs = reinterpret_cast<int4*>(ws);
  int* total = reinterpret_cast<int*>(ws + (int64_t(p.B) * 16 + 255) / 256 * 256);
  hipError_t e = launch_varlen_setup(cu, p.B, p.T, p.H, CK, seqs, nullptr, total, nullptr, stream);
  if (e != hipSuccess) return e;
  p.seqs = seqs;
  return launch_bwd(p, g, ws + bwd_tables_bytes(p.B), stream);
}

// Gradients through the chunk path: workspace = the forward's workspace (its packets, in the
// general-gate or symmetric layout; packed sequences: and the tables) | o (bf16, unused) |
// chunk-start states | chunk-end adjoints (fp16 [dk][dv] per chunk) | M (one gate, FG2: delta) and
// Z (fp16 [C][dv] per chunk) | A_kk (one gate) | the per-token sums of the gradient kernels.
struct BwdChunkedLayout {
  int64_t pkt, obuf, ckS, ckG, ckM, ckZ, ckA, work, total;  // byte offsets
  BwdChunkedLayout(const Problem& p, bool packed) {
    auto up = [](int64_t n) { return (n + 255) / 256 * 256; };
    const int64_t bth = packed ? int64_t(p.T) * p.H : int64_t(p.B) * p.T * p.H;
    const int64_t chunks = packed ? int64_t(p.H) * varlen_max_chunks(p.B, p.T)
                                  : int64_t(p.B) * p.H * ((int64_t(p.T) + CK - 1) / CK);
    const bool one_gate = p.symmetric && !p.rate_sqrt;
    pkt = 0;
    obuf = up(int64_t(packed ? chunk128_varlen_workspace_bytes(p.B, p.T, p.H, p.symmetric, p.decay_channel,
                                                               p.rate_sqrt)
                             : chunk128_workspace_bytes(p.B, p.T, p.H, p.symmetric, p.decay_channel, p.rate_sqrt)));
    ckS = obuf + up(bth * p.dv * 2);
    ckG = ckS + up(chunks * p.dk * p.dv * 2);
    ckM = ckG + up(chunks * p.dk * p.dv * 2);
    ckZ = ckM + up(chunks * CK * p.dv * 2);
    ckA = ckZ + up(chunks * CK * p.dv * 2);
    work = ckA + (one_gate ? up(chunks * 6 * 1024) : 0);
    total = work + up(int64_t(chunk_grad_work_bytes(p, packed)));
  }
};

size_t bwd_chunked_workspace_bytes(const Problem& p) { return size_t(BwdChunkedLayout(p, false).total); }
size_t bwd_chunked_varlen_workspace_bytes(const Problem& p) { return size_t(BwdChunkedLayout(p, true).total); }

namespace {
hipError_t bwd_chunked(const Problem& p, const int* cu, const BwdArgs& g, void* workspace, hipStream_t stream) {
  if (p.dk != 128 || p.dv != 128) return hipErrorInvalidValue;
  const bool packed = cu != nullptr;
  const BwdChunkedLayout L(p, packed);
  char* ws = static_cast<char*>(workspace);
  // The forward stores every chunk's incoming state and its in-chunk reads M (general gates) or
  // delta (one per-head gate, with the prep's A_kk, from which the gradients rebuild M; FG2's
  // rate, whose adjoints need only delta).
  Problem pf = p;
  pf.o = ws + L.obuf;
  pf.o_bf16 = 1;
  pf.S_T = nullptr;
  pf.ck_S = ws + L.ckS;
  pf.ck_M = ws + L.ckM;
  if (p.symmetric && !p.rate_sqrt) pf.ck_A = ws + L.ckA;
  hipError_t e = packed ? launch_chunk128_varlen(pf, cu, ws + L.pkt, stream) : launch_chunk128(pf, ws + L.pkt, stream);
  if (e != hipSuccess) return e;
  if (packed) chunk128_varlen_tables(pf, ws + L.pkt);
  // the state's adjoint at every chunk end and Z, and dS0
  Problem pa = pf;
  pa.ck_S = nullptr;
  pa.ck_M = nullptr;
  pa.ck_A = nullptr;
  pa.ck_G = ws + L.ckG;
  pa.ck_Z = ws + L.ckZ;
  e = launch_chunk128_adjoint(pa, ws + L.pkt, g.dO, g.dS_T, g.dS0, stream);
  if (e != hipSuccess) return e;
  // every chunk's gradients
  Problem pg = pf;
  pg.ck_G = pa.ck_G;
  pg.ck_Z = pa.ck_Z;
  return launch_chunk_grad(pg, g, ws + L.pkt, ws + L.work, stream);
}
}  // namespace

hipError_t launch_bwd_chunked(const Problem& p, const BwdArgs& g, void* workspace, hipStream_t stream) {
  if (p.seqs) return hipErrorInvalidValue;
  return bwd_chunked(p, nullptr, g, workspace, stream);
}

hipError_t launch_bwd_chunked_varlen(const Problem& p, const int* cu, const BwdArgs& g, void* workspace,
                                     hipStream_t stream) {
  return bwd_chunked(p, cu, g, workspace, stream);
}

hipError_t launch_bwd(const Problem& p, const BwdArgs& g, void* workspace, hipStream_t stream) {
  float* ws = static_cast<float*>(workspace);
  const BwdLayout L(p, p.seqs != nullptr);
  dim3 grid(unsigned(p.B * p.H), unsigned(L.ngroups));
  const dim3 block(unsigned(64 * L.wpg));
  switch (p.dk) {
    case 16: hipLaunchKernelGGL(bwd_token_kernel<16>, grid, block, 0, stream, p, g, ws); break;
    case 32: hipLaunchKernelGGL(bwd_token_kernel<32>, grid, block, 0, stream, p, g, ws); break;
    case 64: hipLaunchKernelGGL(bwd_token_kernel<64>, grid, block, 0, stream, p, g, ws); break;
    case 128: hipLaunchKernelGGL(bwd_token_kernel<128>, grid, block, 0, stream, p, g, ws); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(unsigned(L.bth)), dim3(128), 0, stream, p, g, ws + L.parts,
                     ws + L.tmp_dw, L.ngroups, L.bth);
  return hipGetLastError();
}

}  // namespace dr
