/*
 * dr.h -- C ABI of the gated delta-rule recurrence library (libdr.so, gfx950).
 *
 * The operation.  Per batch b and head h a fixed-size associative memory S (dk x dv, fp32)
 * replaces a growing key/value cache; each token decays it, erases along the current key and
 * writes a new key/value association, and the output reads the updated memory
 * ("KronLSTM ...", The problem; "Gated DeltaNet-2: decoupling erase and write in linear
 * attention", the solution and its gate table; "FG2-GDN: Enhancing Long-Context Gated Delta
 * Networks with Doubly Fine-Grained Control", section 2, update rule and FG2-GDN+):
 *
 *     S'  = Diag(a_t) S_{t-1},            a_t = exp(log_decay_t)   (log-space decay, <= 0)
 *     S_t = S' - (e_t * k_t)(k_t^T S') + k_t (w_t * v_t)^T          (erase e_t, write w_t)
 *     o_t = S_t^T q_t
 *
 * Scalar-gate Gated DeltaNet is a per-head decay with e_t = w_t = beta_t; KDA is a per-channel
 * decay with e_t = w_t = beta_t; Gated DeltaNet-2 / FG2-GDN+ use per-channel erase and write
 * gates.  FG2-GDN's symmetric per-channel rate (k~ = sqrt(beta) k, v~ = sqrt(beta) v) is
 * reached by passing the pre-scaled k and v with erase = write = 1.  The operation applies no
 * query scale and no key normalisation: the caller supplies them.
 *
 * Layouts (row-major, contiguous, no strides):
 *     q, k      [B, T, H, dk]        qkv_dtype (fp32 or bf16)
 *     v         [B, T, H, dv]        qkv_dtype
 *     o         [B, T, H, dv]        o_dtype (fp32 default, or bf16)
 *     log_decay [B, T, H] (DR_GATE_HEAD) or [B, T, H, dk] (DR_GATE_CHANNEL), fp32
 *     erase     [B, T, H] or [B, T, H, dk], fp32
 *     write     [B, T, H] or [B, T, H, dv], fp32; ignored when write_is_erase != 0
 *     S0, S_T   [B, H, dk, dv], fp32
 *
 * Ownership and threading.  Every pointer is a device pointer that the caller allocated and
 * keeps alive until the enqueued work has finished.  The library allocates nothing, never
 * synchronises and enqueues all work on `stream` (a hipStream_t; NULL = the default stream),
 * so calls on distinct streams may run concurrently.  Its only global state is the fixed
 * scratch of dr_chunk_fwd_noalloc (a device array per device, and that array's address,
 * resolved once per device).
 *
 * Range.  The matrix-core path multiplies fp16 operands: q, k, v and the fp32 state enter its
 * products as fp16, so entries of q, k, v or S of magnitude 65504 or more (and values formed
 * from them, such as beta (v - S^T k)) overflow there.  Decay factors never do: every one is
 * at most one, or bounded by e^6 where the inputs are checked to be moderate, for any decay in
 * (0, 1].  The token-by-token path (fp32) has no such limit.
 *
 * Errors.  Argument errors are detected synchronously, before anything is enqueued, and the
 * call returns a negative dr_status with no device work issued.  A failed launch returns
 * DR_E_HIP.  Faults inside a kernel surface at the caller's next synchronisation.  NaN and Inf
 * inputs are not checked; they stay inside the (b, h) they occur in.
 */
#ifndef GATED_DELTA_RULE_DR_H_
#define GATED_DELTA_RULE_DR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DR_ABI_VERSION 1

/* Status codes returned by every entry point. */
typedef enum {
  DR_OK = 0,
  DR_E_NULL = -1,        /* a required pointer (or the descriptor) is NULL */
  DR_E_SHAPE = -2,       /* a size is negative, zero where it must not be, or overflows */
  DR_E_DTYPE = -3,       /* unknown dtype or gate-kind code */
  DR_E_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  DR_E_ALIAS = -5,       /* an output overlaps an input (other than the allowed S0 == S_T) */
  DR_E_UNSUPPORTED = -6, /* a valid combination this library does not implement */
  DR_E_WORKSPACE = -7,   /* workspace missing or smaller than dr_chunk_fwd_workspace_bytes */
  DR_E_HIP = -8,         /* a HIP launch failed */
  DR_E_SCRATCH = -9      /* dr_chunk_fwd_noalloc: the problem needs more workspace than its fixed
                            scratch holds (dr_chunk_fwd_noalloc_max_bytes) */
} dr_status;

typedef enum { DR_F32 = 0, DR_BF16 = 1 } dr_dtype;

typedef enum {
  DR_GATE_HEAD = 0,     /* one fp32 value per (b, t, h): [B, T, H] */
  DR_GATE_CHANNEL = 1,  /* one fp32 value per channel: [B, T, H, dk] (decay, erase) or dv (write) */
  DR_GATE_RATE_SQRT = 2 /* erase only: FG2-GDN's per-channel learning rate beta [B, T, H, dk],
                           absorbed symmetrically into key and value, k~ = sqrt(beta) * k and
                           v~ = sqrt(beta) * v, after which the update erases and writes with the
                           unit gate: S_t = (I - k~ k~^T) Diag(a_t) S_{t-1} + k~ v~^T ("FG2-GDN
                           ...", section 2, FG2-GDN update rule).  Needs write_is_erase != 0
                           (DR_E_DTYPE otherwise) and dk == dv (DR_E_SHAPE otherwise); q is not
                           scaled. */
} dr_gate_kind;

/* Problem descriptor.  All fields are 32-bit integers so the struct has one layout on every
 * compiler: 12 x int32, no padding. */
typedef struct {
  int32_t B, T, H;        /* batch, tokens (T >= 0), heads */
  int32_t dk, dv;         /* key and value widths: each one of 16, 32, 64, 128 */
  int32_t chunk;          /* dr_chunk_fwd: 0 = default (64); 1 = token-by-token path; else 64 */
  int32_t qkv_dtype;      /* dr_dtype of q, k, v */
  int32_t o_dtype;        /* dr_dtype of o (DR_F32 recommended) */
  int32_t decay_kind;     /* dr_gate_kind of log_decay */
  int32_t erase_kind;     /* dr_gate_kind of erase */
  int32_t write_kind;     /* dr_gate_kind of write (ignored when write_is_erase) */
  int32_t write_is_erase; /* nonzero: the write gate is the erase gate (`write` is ignored);
                             with a per-channel erase gate this needs dk == dv */
} dr_desc;

/* Returns DR_ABI_VERSION of the built library. */
int dr_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* dr_status_str(int status);

/* Bytes of device workspace dr_chunk_fwd needs for `desc` (0 when none), or 0 for an invalid
 * descriptor.  The matrix-core path stores, per 64-token chunk of every (b, h), one packet of
 * the chunk's state-independent factors: the triangular-solve factor and the in-chunk
 * decay-weighted Gram matrices (lower-triangular fp16 64 x 64, only their six nonzero 16 x 32
 * blocks), the gate factors, and the fp16 key/query tiles (decayed from the chunk start, plus
 * the keys decayed to the chunk end, unless the decay is per head with one per-head gate for
 * erase and write).  That is
 * B * H * ceil(T / 64) * P bytes with P = 46080 (per-head decay, one per-head erase/write gate),
 * 63488 (per-channel decay, one per-head erase/write gate), 62464 (per-head decay,
 * DR_GATE_RATE_SQRT) or 79872 (per-channel decay, DR_GATE_RATE_SQRT; these two add the scaled
 * values v~ as fp16 [64][128]) or 92160 (otherwise); with separate erase and write gates
 * that count is rounded up to a multiple of 256 and followed by the segment maps of the
 * segmented scan: B * H * S * 196608 bytes (fp32 F, H and the entering state per segment), where
 * S = 1 + min(256 / (B * H), 8) segments, at most half the chunk count, and no maps when S is 1
 * (B * H >= 256, or fewer than four chunks).  The
 * token-by-token path needs none.  The caller allocates it
 * (any device memory, 16-byte aligned, not overlapping the other arguments) and may reuse it
 * once the call's work has finished. */
size_t dr_chunk_fwd_workspace_bytes(const dr_desc* desc);

/* Prefill / training forward over T tokens (the chunkwise-parallel form the pages describe:
 * the in-chunk rank-1 erases are folded into dense products via a triangular solve (WY/UT),
 * and the fp32 state is carried from chunk to chunk).
 *
 *   S0    initial state, or NULL for zeros.  May be the same pointer as S_T (in-place carry);
 *         any other overlap between S0 and S_T is DR_E_ALIAS.
 *   o     output; must not overlap any input or S_T.
 *   S_T   final state, or NULL to skip writing it.
 *   workspace, workspace_bytes: device scratch of at least dr_chunk_fwd_workspace_bytes(desc)
 *         (NULL / 0 when that is 0).
 * T == 0 leaves o untouched and writes S_T = S0 (zeros when S0 is NULL).
 * Paths: bf16 q/k/v with dk == dv == 128 and chunk 0/64 run the MFMA chunk kernel (fp16
 * operands, fp32 accumulation and fp32 state); every other supported combination, and
 * chunk == 1, runs the fp32 token-by-token kernel.
 * Pointers must be 16-byte aligned. */
int dr_chunk_fwd(const dr_desc* desc, const void* q, const void* k, const void* v,
                 const float* log_decay, const float* erase, const float* write,
                 const float* S0, void* o, float* S_T, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same operation, paths,
 * arguments and errors as dr_chunk_fwd without the workspace arguments: the workspace is a
 * fixed device array inside the library (dr_chunk_fwd_noalloc_max_bytes() = 64 MiB), one per
 * device, allocated when the library's device code is loaded on that device and held until the
 * process ends; the call itself allocates nothing.  A problem whose dr_chunk_fwd_workspace_bytes
 * exceeds it returns DR_E_SCRATCH before any device work (by gate kind, about 840 to 1,450
 * chunks of 64 tokens across all (b, h) with one erase/write gate; with separate erase and write
 * gates up to 728 chunks when B * H >= 256, and for fewer heads less because of the segment maps:
 * e.g. H = 32 heads of up to 704 tokens).  All calls on one device share its array: calls
 * that may overlap in time on one device (different streams, or different host threads without
 * ordering) race and must be serialised by the caller.  Nothing in the array needs clearing between calls (each call
 * writes every byte it reads).  The first call on a device resolves the array's device
 * address (hipGetSymbolAddress); a failure there returns DR_E_HIP. */
size_t dr_chunk_fwd_noalloc_max_bytes(void);

int dr_chunk_fwd_noalloc(const dr_desc* desc, const void* q, const void* k, const void* v,
                         const float* log_decay, const float* erase, const float* write,
                         const float* S0, void* o, float* S_T, void* stream);

/* Packed batches of sequences of different lengths (serving prefill).  The nseq sequences lie
 * one after another on the token axis of the dr_chunk_fwd layouts with B = 1 (desc->B must be
 * 1 and desc->T is the packed token count): sequence n holds tokens cu_seqlens[n] ..
 * cu_seqlens[n + 1] - 1.  Each sequence is an independent recurrence with its own state, as
 * a server holds one fixed-size state per conversation ("Gated DeltaNet-2: decoupling erase
 * and write in linear attention", sections "The attention bottleneck" and "Why this matters":
 * constant-size state, constant-memory decoding); the packed layout is this library's own
 * convention (those sections describe none).
 *
 *   cu_seqlens  nseq + 1 int32 offsets in device memory, 4-byte aligned, read on the device
 *               (so the call cannot check them).  Valid offsets start at 0, never decrease and
 *               end at desc->T.  The kernels clamp every offset into [0, T] and take the
 *               running maximum, so no access leaves the arrays whatever they hold: the
 *               results for invalid offsets are those of the offsets so corrected, and tokens
 *               outside every sequence leave o untouched.
 *   S0, S_T     [nseq, H, dk, dv] fp32 (S0 NULL = zeros, S_T NULL = skip; S0 may equal S_T).
 *               An empty sequence writes S_T[n] = S0[n] (zeros without S0).  S_T is the state
 *               layout of dr_decode_step with B = nseq, so decoding continues from it directly.
 *   workspace   at least dr_chunk_fwd_varlen_workspace_bytes(desc, nseq) bytes.
 * The paths are those of dr_chunk_fwd.  nseq == 0 or T == 0 enqueues at most the S_T copy.
 * Errors as dr_chunk_fwd; nseq < 0 or > 2^30 is DR_E_SHAPE, a NULL cu_seqlens with nseq > 0
 * DR_E_NULL, a cu_seqlens not 4-byte aligned DR_E_ALIGN, and cu_seqlens overlapping an
 * output or the workspace DR_E_ALIAS. */

/* Workspace bytes of dr_chunk_fwd_varlen (0 for an invalid descriptor or nseq).  The
 * matrix-core path keeps the packets of dr_chunk_fwd for at most floor((T + 63 nseq) / 64)
 * chunks per head (P bytes each, P as above), plus tables of 16 bytes per chunk and 20 bytes
 * per sequence (each table rounded up to 256 bytes) and 256 bytes; the token-by-token path
 * needs the 16-byte sequence table and 256 bytes only. */
size_t dr_chunk_fwd_varlen_workspace_bytes(const dr_desc* desc, int32_t nseq);

int dr_chunk_fwd_varlen(const dr_desc* desc, const int32_t* cu_seqlens, int32_t nseq, const void* q,
                        const void* k, const void* v, const float* log_decay, const float* erase,
                        const float* write, const float* S0, void* o, float* S_T, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Gradients for training: of L = sum(o * dO) + sum(S_T * dS_T) with respect to every input of
 * dr_chunk_fwd ("FG2-GDN ...", sections 2-3: the WY form makes training chunk-parallel;
 * "Linearized 2-Simplicial Attention", method: the backward is a second scan over the chunks).
 * Two paths:
 *   - bf16 q/k/v with dk == dv == 128 and chunk 0 or 64 (the matrix-core path; dense or packed
 *     with dr_chunk_bwd_varlen): the chunked
 *     forward runs again and stores every chunk's incoming state and in-chunk reads, a reverse
 *     scan over the chunks carries the state's adjoint and stores it at every chunk end, and
 *     per-chunk kernels form the gradients on the matrix cores (fp16 operands, fp32
 *     accumulation; the forward's accuracy);
 *   - everything else, and chunk == 1: the fp32 adjoint of the token loop (state checkpoints
 *     every 64 tokens, the tokens walked backwards).
 *
 *   dO     [B, T, H, dv] fp32 (required).       dS_T  [B, H, dk, dv] fp32, or NULL for zero.
 *   dq, dk [B, T, H, dk] fp32; dv [B, T, H, dv] fp32 (all required).
 *   dlog_decay, derase, dwrite: fp32 in the layouts of log_decay, erase and write (a per-head
 *          gate gets the sum over its channels).  With write_is_erase the one gate's gradient
 *          (both uses) goes to derase and dwrite is ignored.
 *   dS0    [B, H, dk, dv] fp32, or NULL to skip.
 *   workspace: at least dr_chunk_bwd_workspace_bytes(desc) bytes.  Matrix-core path: the
 *          forward's packets, a bf16 copy of o, per 64-token chunk the incoming state and its
 *          adjoint at the chunk end (fp16, 32 KB each), the reads and Z (fp16, 16 KB each), with
 *          one per-head gate A_kk (6 KB), and 1.6 KB of per-token sums per chunk.
 *          Token path: a state checkpoint every 64 tokens and one chunk of states per (b, h,
 *          group of 256 / dk value columns), and four fp32 partial sums per row for every 32
 *          value columns (at dk = dv = 128, 8 KB per token and head).
 * Outputs must not overlap one another, any input or the workspace.  T == 0 writes dS0 = dS_T
 * (zeros without it).  With DR_GATE_RATE_SQRT, derase is the gradient of the rate beta (through
 * both sqrt(beta) k and sqrt(beta) v).  Errors as dr_chunk_fwd. */
size_t dr_chunk_bwd_workspace_bytes(const dr_desc* desc);

int dr_chunk_bwd(const dr_desc* desc, const void* q, const void* k, const void* v,
                 const float* log_decay, const float* erase, const float* write, const float* S0,
                 const float* dO, const float* dS_T, float* dq, float* dk, float* dv,
                 float* dlog_decay, float* derase, float* dwrite, float* dS0, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Gradients over a packed batch of nseq sequences (the layouts and offsets of
 * dr_chunk_fwd_varlen; desc->B must be 1): every gradient as dr_chunk_bwd, with S0, dS_T and dS0
 * [nseq, H, dk, dv].  The offsets are clamped as for dr_chunk_fwd_varlen; gradient rows of
 * tokens in no sequence (possible only with invalid offsets) are left unspecified.  Errors as
 * dr_chunk_bwd plus those of the offsets as in dr_chunk_fwd_varlen. */
size_t dr_chunk_bwd_varlen_workspace_bytes(const dr_desc* desc, int32_t nseq);

int dr_chunk_bwd_varlen(const dr_desc* desc, const int32_t* cu_seqlens, int32_t nseq, const void* q,
                        const void* k, const void* v, const float* log_decay, const float* erase,
                        const float* write, const float* S0, const float* dO, const float* dS_T,
                        float* dq, float* dk, float* dv, float* dlog_decay, float* derase,
                        float* dwrite, float* dS0, void* workspace, size_t workspace_bytes,
                        void* stream);

/* One decode token for B independent sequences (desc->T must be 1): reads q, k, v, gates in
 * the [B, 1, H, d] layouts above, updates S [B, H, dk, dv] in place and writes o [B, 1, H, dv].
 * The state streams through once (read once, written once).  o must not overlap any input
 * or S.  Pointers must be 16-byte aligned. */
int dr_decode_step(const dr_desc* desc, const void* q, const void* k, const void* v,
                   const float* log_decay, const float* erase, const float* write, float* S,
                   void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GATED_DELTA_RULE_DR_H_ */
