// Internal launch interface between the C-ABI layer (dr_api.cpp) and the kernels.
// Every launcher enqueues on `stream`, never synchronises and returns the hipError_t of the
// launch.  Arguments have been validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

// One problem, already validated.  Gate pointers may be per head or per channel.
struct Problem {
  int B, T, H, dk, dv;
  int qkv_bf16;        // 1: q, k, v are bf16; 0: fp32
  int o_bf16;          // 1: o is bf16; 0: fp32
  int decay_channel;   // log_decay is [B,T,H,dk]
  int erase_channel;   // erase is [B,T,H,dk]
  int write_channel;   // write is [B,T,H,dv]
  int symmetric;       // one per-head gate is both erase and write (write is erase)
  int rate_sqrt;       // erase is a per-channel rate beta absorbed as sqrt(beta) into k and v
                       // (the update then erases and writes with the unit gate); write is erase
  const void* q;
  const void* k;
  const void* v;
  const float* log_decay;
  const float* erase;
  const float* write;  // == erase when the write gate is the erase gate
  const float* S0;     // may be null (zeros)
  void* o;
  float* S_T;          // may be null (skip)
  // Packed sequences of different lengths: B is then the number of sequences and T the
  // packed token count, and the kernels take each sequence's tokens from these tables (in the
  // workspace, written by launch_varlen_setup).  Null for a dense [B, T] batch.
  const int4* seqs = nullptr;          // [B] {first token, tokens, H * chunks before, chunks}
  const int4* chunks = nullptr;        // [chunks] {first token, tokens, packet of head 0, chunks
                                       //  of its sequence}; the packet of head h adds h * chunks
  const int* nchunks_total = nullptr;  // number of entries in `chunks`
  const int* order = nullptr;          // [B] sequences, longest first (scan workgroup order)
  // Gradients through the chunk path: the state at the start of every chunk (forward scans) and
  // its adjoint at the end of every chunk (adjoint scan), fp16 [packet][dv / 16][dk][16] (16-column
  // tiles, each a contiguous 4 KB, so that the scans write whole lines); null otherwise.
  void* ck_S = nullptr;
  void* ck_G = nullptr;
  // ... and, as fp16 [packet][dv / 16][token][16], the forward's in-chunk reads M (general gates;
  // with one gate or FG2's rate the symmetric scan's delta instead) and the adjoint scan's Z (the
  // adjoint of K+ S + A_kk Vt); null otherwise.
  void* ck_M = nullptr;
  void* ck_Z = nullptr;
  // ... and with one per-head gate, the prep's A_kk (fp16, the packet's six-block triangular
  // layout, 6 KB per chunk), from which the gradients rebuild M; null otherwise.
  void* ck_A = nullptr;
};

// Sequence tables of a packed batch (one workgroup): from nseq + 1 device offsets `cu` over T
// packed tokens, clamped into [0, T] and made nondecreasing, writes seqs[nseq], chunks[] (when
// not null; at most varlen_max_chunks entries), *total, for chunks of `chunk` tokens, and
// (when not null) order[nseq], the sequences longest first.
hipError_t launch_varlen_setup(const int* cu, int nseq, int T, int H, int chunk, int4* seqs, int4* chunks,
                               int* total, int* order, hipStream_t stream);

// Upper bound on the chunks of nseq sequences with T tokens in all: sum ceil(len / 64).
__host__ __device__ inline int64_t varlen_max_chunks(int64_t nseq, int64_t T) { return (T + 63 * nseq) / 64; }

// fp32 token-by-token recurrence: any supported dk/dv/dtypes.  Reads S0 before writing S_T
// element by element in the same thread, so S0 == S_T is safe.
hipError_t launch_recurrent(const Problem& p, hipStream_t stream);

// Single-token decode with the state updated in place (S0 == S_T == S), dk == dv == 128.
hipError_t launch_decode128(const Problem& p, hipStream_t stream);

// MFMA chunked forward, bf16 q/k/v, dk == dv == 128, chunk 64.  `workspace` holds at least
// chunk128_workspace_bytes(B, T, H, symmetric, decay_channel, rate_sqrt) bytes: one packet of
// state-independent factors per chunk of every (b, h).
size_t chunk128_workspace_bytes(int B, int T, int H, bool symmetric, bool decay_channel, bool rate_sqrt);
hipError_t launch_chunk128(const Problem& p, void* workspace, hipStream_t stream);
// The full-width segmented scan of separate erase and write gates over a dense batch (after the
// prep has written the packets at `ws`): `extra` holds wide_workspace_bytes(B, T, H) bytes for
// the segments' maps and entering states (null when that is 0).
size_t wide_workspace_bytes(int B, int T, int H);
hipError_t launch_scan_wide(const Problem& p, const char* ws, float* extra, hipStream_t stream);
// The same segmentation for the gradients' adjoint scan (general gates, dense batch): G and Z of
// every chunk into p.ck_G, p.ck_Z, dS0 (when not null), from dO and dS_T (null: zero).
hipError_t launch_adjoint_wide(const Problem& p, const char* ws, float* extra, const float* dO, const float* dS_T,
                               float* dS0, hipStream_t stream);

// The adjoint scan over the packets that launch_chunk128 left in `workspace` (same problem): the
// state's adjoint at the end of every chunk into p.ck_G and at the start of the sequence into
// dS0 (when not null), from dO [B,T,H,dv] and dS_T (null: zero).
// The table pointers (p.seqs, p.chunks, p.nchunks_total, p.order) of a packed batch in the
// workspace of launch_chunk128_varlen (the tables its setup kernel writes).
void chunk128_varlen_tables(Problem& p, void* workspace);
hipError_t launch_chunk128_adjoint(const Problem& p, const void* workspace, const float* dO, const float* dS_T,
                                   float* dS0, hipStream_t stream);

// The same over p.B packed sequences delimited by the device offsets `cu` (p.B + 1 of them):
// the workspace holds the packets of at most varlen_max_chunks(p.B, p.T) chunks per head,
// then the sequence tables.
size_t chunk128_varlen_workspace_bytes(int nseq, int T, int H, bool symmetric, bool decay_channel, bool rate_sqrt);
hipError_t launch_chunk128_varlen(Problem p, const int* cu, void* workspace, hipStream_t stream);

// The token-by-token kernel over packed sequences: the workspace holds the sequence table.
size_t recurrent_varlen_workspace_bytes(int nseq);
hipError_t launch_recurrent_varlen(Problem p, const int* cu, void* workspace, hipStream_t stream);

// Gradients of the recurrence (fp32 adjoint of the token loop; any supported width).  The
// outputs are fp32 in their inputs' layouts; dwrite is null when the write gate is the erase
// gate (derase then takes both parts); dS_T and dS0 may be null.
struct BwdArgs {
  const float* dO;    // [B, T, H, dv]
  const float* dS_T;  // [B, H, dk, dv] or null (zero)
  float* dq;
  float* dk;
  float* dv;
  float* dlog_decay;
  float* derase;
  float* dwrite;
  float* dS0;
};
size_t bwd_workspace_bytes(const Problem& p);
hipError_t launch_bwd(const Problem& p, const BwdArgs& g, void* workspace, hipStream_t stream);
// Gradients through the matrix-core chunk path (bf16 q/k/v, dk == dv == 128, a dense batch): the
// chunked forward stores every chunk's incoming state and in-chunk reads, the adjoint scan every
// chunk's end adjoint and Z, and each chunk's gradients then follow on the matrix cores.
size_t bwd_chunked_workspace_bytes(const Problem& p);
hipError_t launch_bwd_chunked(const Problem& p, const BwdArgs& g, void* workspace, hipStream_t stream);
// The same over p.B packed sequences delimited by the device offsets `cu` (p.T packed tokens).
size_t bwd_chunked_varlen_workspace_bytes(const Problem& p);
hipError_t launch_bwd_chunked_varlen(const Problem& p, const int* cu, const BwdArgs& g, void* workspace,
                                     hipStream_t stream);
// The per-chunk gradient kernels (p carries ck_S, ck_G, ck_M, ck_Z (and ck_A), and for packed
// sequences the chunk tables; `packets` the forward's packets; `work` chunk_grad_work_bytes bytes).
size_t chunk_grad_work_bytes(const Problem& p, bool packed);
hipError_t launch_chunk_grad(const Problem& p, const BwdArgs& g, const void* packets, void* work,
                             hipStream_t stream);
// The same over p.B packed sequences delimited by the device offsets `cu` (p.T packed tokens).
size_t bwd_varlen_workspace_bytes(const Problem& p);
hipError_t launch_bwd_varlen(Problem p, const int* cu, const BwdArgs& g, void* workspace, hipStream_t stream);

// S_T = S0 (copy) or zeros when S0 is null: n floats.
hipError_t launch_state_copy(const float* S0, float* S_T, int64_t n, hipStream_t stream);

}  // namespace dr
