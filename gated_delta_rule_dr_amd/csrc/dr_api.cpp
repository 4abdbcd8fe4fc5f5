// C-ABI layer of libdr: argument validation, path selection and launch.
//
// Validation is synchronous and touches no HIP API, so every error path can be exercised on
// a host without a GPU; nothing is enqueued unless all checks pass.

#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/dr.h"
#include "dr_internal.h"

namespace {

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Range range_of(const void* p, uint64_t bytes) {
  Range r;
  if (p != nullptr && bytes > 0) {
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + bytes;
  }
  return r;
}

bool overlaps(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_width(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Byte extents of every array of a problem.
struct Extents {
  uint64_t qk, v, o, decay, erase, write, state;
};

// Element counts are bounded so that every index the kernels form fits in int64 and every
// per-(b,h) offset fits in int32 arithmetic where the kernels use it.
constexpr uint64_t kMaxElems = uint64_t(1) << 40;
// Sequences of one packed batch.
constexpr int32_t kMaxSeqs = int32_t(1) << 30;

int check_desc(const dr_desc* d, bool decode, Extents* ex) {
  if (d == nullptr) return DR_E_NULL;
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->dk < 1 || d->dv < 1) return DR_E_SHAPE;
  if (decode && d->T != 1) return DR_E_SHAPE;
  if (d->qkv_dtype != DR_F32 && d->qkv_dtype != DR_BF16) return DR_E_DTYPE;
  if (d->o_dtype != DR_F32 && d->o_dtype != DR_BF16) return DR_E_DTYPE;
  auto kind_ok = [](int k) { return k == DR_GATE_HEAD || k == DR_GATE_CHANNEL; };
  const bool rate = d->erase_kind == DR_GATE_RATE_SQRT;
  if (!kind_ok(d->decay_kind) || !(kind_ok(d->erase_kind) || rate)) return DR_E_DTYPE;
  if (!d->write_is_erase && !kind_ok(d->write_kind)) return DR_E_DTYPE;
  if (rate && !d->write_is_erase) return DR_E_DTYPE;
  if (!supported_width(d->dk) || !supported_width(d->dv)) return DR_E_UNSUPPORTED;
  if (!decode && d->chunk != 0 && d->chunk != 1 && d->chunk != 64) return DR_E_UNSUPPORTED;
  if (d->write_is_erase && d->erase_kind != DR_GATE_HEAD && d->dk != d->dv) return DR_E_SHAPE;

  const uint64_t B = uint64_t(d->B), T = uint64_t(d->T), H = uint64_t(d->H);
  const uint64_t dk = uint64_t(d->dk), dv = uint64_t(d->dv);
  const uint64_t bth = B * T * H;  // < 2^93 impossible: each factor < 2^31, check stepwise
  if (B * H > kMaxElems || (T > 0 && bth / T != B * H) || bth > kMaxElems / 128)
    return DR_E_SHAPE;
  if (B * H * dk * dv > kMaxElems) return DR_E_SHAPE;
  const uint64_t qkv_sz = d->qkv_dtype == DR_BF16 ? 2 : 4;
  const uint64_t o_sz = d->o_dtype == DR_BF16 ? 2 : 4;
  ex->qk = bth * dk * qkv_sz;
  ex->v = bth * dv * qkv_sz;
  ex->o = bth * dv * o_sz;
  ex->decay = bth * (d->decay_kind == DR_GATE_CHANNEL ? dk : 1) * 4;
  ex->erase = bth * (d->erase_kind != DR_GATE_HEAD ? dk : 1) * 4;
  if (d->write_is_erase)
    ex->write = 0;
  else
    ex->write = bth * (d->write_kind == DR_GATE_CHANNEL ? dv : 1) * 4;
  ex->state = B * H * dk * dv * 4;
  return DR_OK;
}

// A required array must be non-null unless it is empty; every non-null pointer is 16-byte
// aligned.
int check_ptr(const void* p, uint64_t bytes, bool required) {
  if (p == nullptr) return (required && bytes > 0) ? DR_E_NULL : DR_OK;
  return aligned16(p) ? DR_OK : DR_E_ALIGN;
}

// One per-head gate serves as both erase and write gate.
bool is_symmetric(const dr_desc* d) { return d->write_is_erase && d->erase_kind == DR_GATE_HEAD; }

dr::Problem make_problem(const dr_desc* d, const void* q, const void* k, const void* v,
                         const float* log_decay, const float* erase, const float* write,
                         const float* S0, void* o, float* S_T) {
  dr::Problem p;
  p.B = d->B;
  p.T = d->T;
  p.H = d->H;
  p.dk = d->dk;
  p.dv = d->dv;
  p.qkv_bf16 = d->qkv_dtype == DR_BF16;
  p.o_bf16 = d->o_dtype == DR_BF16;
  p.decay_channel = d->decay_kind == DR_GATE_CHANNEL;
  p.erase_channel = d->erase_kind != DR_GATE_HEAD;
  p.rate_sqrt = d->erase_kind == DR_GATE_RATE_SQRT;
  p.write_channel = d->write_is_erase ? p.erase_channel : (d->write_kind == DR_GATE_CHANNEL);
  p.q = q;
  p.k = k;
  p.v = v;
  p.log_decay = log_decay;
  p.erase = erase;
  p.write = d->write_is_erase ? erase : write;
  p.symmetric = is_symmetric(d);
  p.S0 = S0;
  p.o = o;
  p.S_T = S_T;
  return p;
}

// The matrix-core path: bf16 q/k/v, dk == dv == 128, chunk 0 or 64, at least one token.
bool uses_chunk128(const dr_desc* d) {
  return d->qkv_dtype == DR_BF16 && d->dk == 128 && d->dv == 128 && d->chunk != 1 && d->T > 0;
}

int launched(hipError_t launch_err) {
  if (launch_err != hipSuccess) return DR_E_HIP;
  return hipGetLastError() == hipSuccess ? DR_OK : DR_E_HIP;
}


size_t chunk_fwd_workspace(const dr_desc* desc);

// Validation of a dense forward call.  check_ws: the caller passes the workspace (it must be
// large enough and must not overlap the other arrays); otherwise the library supplies it.
int check_chunk_fwd(const dr_desc* d, const void* q, const void* k, const void* v, const float* log_decay,
                    const float* erase, const float* write, const float* S0, const void* o, const float* S_T,
                    const void* workspace, size_t workspace_bytes, bool check_ws, Extents* exo) {
  Extents& ex = *exo;
  int st = check_desc(d, false, &ex);
  if (st != DR_OK) return st;
  const bool need_write = !d->write_is_erase;
  if ((st = check_ptr(q, ex.qk, true)) || (st = check_ptr(k, ex.qk, true)) ||
      (st = check_ptr(v, ex.v, true)) || (st = check_ptr(log_decay, ex.decay, true)) ||
      (st = check_ptr(erase, ex.erase, true)) ||
      (st = check_ptr(need_write ? write : nullptr, ex.write, need_write)) ||
      (st = check_ptr(S0, ex.state, false)) || (st = check_ptr(o, ex.o, true)) ||
      (st = check_ptr(S_T, ex.state, false)) || (st = check_ptr(workspace, workspace_bytes, false)))
    return st;
  if (check_ws && workspace_bytes < chunk_fwd_workspace(d)) return DR_E_WORKSPACE;

  const Range rin[] = {range_of(q, ex.qk),         range_of(k, ex.qk),
                       range_of(v, ex.v),          range_of(log_decay, ex.decay),
                       range_of(erase, ex.erase),  range_of(need_write ? write : nullptr, ex.write),
                       range_of(S0, ex.state)};
  const Range ro = range_of(o, ex.o), rs = range_of(S_T, ex.state);
  for (const Range& r : rin)
    if (overlaps(ro, r)) return DR_E_ALIAS;
  if (overlaps(ro, rs)) return DR_E_ALIAS;
  for (int i = 0; i < 6; ++i)
    if (overlaps(rs, rin[i])) return DR_E_ALIAS;
  if (S0 != nullptr && S_T != nullptr && S0 != S_T && overlaps(rs, rin[6])) return DR_E_ALIAS;
  if (check_ws) {
    const Range rw = range_of(workspace, workspace_bytes);
    for (const Range& r : rin)
      if (overlaps(rw, r)) return DR_E_ALIAS;
    if (overlaps(rw, ro) || overlaps(rw, rs)) return DR_E_ALIAS;
  }
  return DR_OK;
}

// Launch of a validated dense forward call.
int launch_chunk_fwd(const dr_desc* d, const void* q, const void* k, const void* v, const float* log_decay,
                     const float* erase, const float* write, const float* S0, void* o, float* S_T, void* workspace,
                     const Extents& ex, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d->T == 0) {
    if (S_T == nullptr || S_T == S0) return DR_OK;
    return launched(dr::launch_state_copy(S0, S_T, int64_t(ex.state / 4), s));
  }
  dr::Problem p = make_problem(d, q, k, v, log_decay, erase, write, S0, o, S_T);
  if (uses_chunk128(d)) return launched(dr::launch_chunk128(p, workspace, s));
  return launched(dr::launch_recurrent(p, s));
}

// ---- the fixed scratch of dr_chunk_fwd_noalloc -------------------------------------------
// A file-scope device array (each device that loads the library holds its own copy until the
// process ends).  Host code never uses the array's name as an address: it is a host-side
// stand-in.  The device address is resolved once per device, with that device current, by
// hipGetSymbolAddress, and only that address reaches kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// This device's scratch address (the current device).
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DR_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DR_E_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return DR_E_HIP;
  *out = g_scratch_ptr[dev];
  return DR_OK;
}

// Validation and launch of the gradient call, dense (packed == false) or over nseq packed
// sequences delimited by cu_seqlens (packed == true: desc->B == 1, states [nseq, H, dk, dv]).
int chunk_bwd_common(const dr_desc* d, const int32_t* cu_seqlens, int32_t nseq, bool packed, const void* q,
                     const void* k, const void* v, const float* log_decay, const float* erase, const float* write,
                     const float* S0, const float* dO, const float* dS_T, float* dq, float* dk, float* dv,
                     float* dlog_decay, float* derase, float* dwrite, float* dS0, void* workspace,
                     size_t workspace_bytes, void* stream);

}  // namespace

extern "C" {

int dr_abi_version(void) { return DR_ABI_VERSION; }

const char* dr_status_str(int status) {
  switch (status) {
    case DR_OK: return "ok";
    case DR_E_NULL: return "a required pointer or the descriptor is NULL";
    case DR_E_SHAPE: return "invalid or overflowing size";
    case DR_E_DTYPE: return "unknown dtype or gate kind";
    case DR_E_ALIGN: return "pointer not 16-byte aligned";
    case DR_E_ALIAS: return "an output overlaps an input";
    case DR_E_UNSUPPORTED: return "combination not supported by this library";
    case DR_E_WORKSPACE: return "workspace missing or too small";
    case DR_E_HIP: return "HIP launch failed";
    case DR_E_SCRATCH: return "the problem needs more than the fixed scratch of dr_chunk_fwd_noalloc";
    default: return "unknown status";
  }
}

size_t dr_chunk_fwd_workspace_bytes(const dr_desc* desc) { return chunk_fwd_workspace(desc); }

}  // extern "C"

namespace {
size_t chunk_fwd_workspace(const dr_desc* desc) {
  Extents ex;
  if (check_desc(desc, false, &ex) != DR_OK) return 0;
  if (!uses_chunk128(desc)) return 0;
  return dr::chunk128_workspace_bytes(desc->B, desc->T, desc->H, is_symmetric(desc),
                                      desc->decay_kind == DR_GATE_CHANNEL,
                                      desc->erase_kind == DR_GATE_RATE_SQRT);
}
}  // namespace

extern "C" {

int dr_chunk_fwd(const dr_desc* d, const void* q, const void* k, const void* v,
                 const float* log_decay, const float* erase, const float* write,
                 const float* S0, void* o, float* S_T, void* workspace, size_t workspace_bytes,
                 void* stream) {
  Extents ex;
  const int st = check_chunk_fwd(d, q, k, v, log_decay, erase, write, S0, o, S_T, workspace, workspace_bytes,
                                 true, &ex);
  if (st != DR_OK) return st;
  return launch_chunk_fwd(d, q, k, v, log_decay, erase, write, S0, o, S_T, workspace, ex, stream);
}

size_t dr_chunk_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int dr_chunk_fwd_noalloc(const dr_desc* d, const void* q, const void* k, const void* v,
                         const float* log_decay, const float* erase, const float* write,
                         const float* S0, void* o, float* S_T, void* stream) {
  Extents ex;
  int st = check_chunk_fwd(d, q, k, v, log_decay, erase, write, S0, o, S_T, nullptr, 0, false, &ex);
  if (st != DR_OK) return st;
  const size_t need = dr_chunk_fwd_workspace_bytes(d);
  if (need > kScratchBytes) return DR_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_ptr(&ws)) != DR_OK) return st;
  return launch_chunk_fwd(d, q, k, v, log_decay, erase, write, S0, o, S_T, ws, ex, stream);
}

size_t dr_chunk_fwd_varlen_workspace_bytes(const dr_desc* desc, int32_t nseq) {
  Extents ex;
  if (check_desc(desc, false, &ex) != DR_OK || desc->B != 1 || nseq <= 0 || nseq > kMaxSeqs) return 0;
  if (uses_chunk128(desc))
    return dr::chunk128_varlen_workspace_bytes(nseq, desc->T, desc->H, is_symmetric(desc),
                                               desc->decay_kind == DR_GATE_CHANNEL,
                                               desc->erase_kind == DR_GATE_RATE_SQRT);
  return dr::recurrent_varlen_workspace_bytes(nseq);
}

int dr_chunk_fwd_varlen(const dr_desc* d, const int32_t* cu_seqlens, int32_t nseq, const void* q,
                        const void* k, const void* v, const float* log_decay, const float* erase,
                        const float* write, const float* S0, void* o, float* S_T, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Extents ex;
  int st = check_desc(d, false, &ex);
  if (st != DR_OK) return st;
  if (d->B != 1 || nseq < 0 || nseq > kMaxSeqs) return DR_E_SHAPE;
  // the states are [nseq, H, dk, dv]
  const uint64_t state_elems = uint64_t(nseq) * uint64_t(d->H) * uint64_t(d->dk) * uint64_t(d->dv);
  if (state_elems > kMaxElems) return DR_E_SHAPE;
  ex.state = state_elems * 4;
  const uint64_t cu_bytes = (uint64_t(nseq) + 1) * 4;
  if (cu_seqlens == nullptr) {
    if (nseq > 0) return DR_E_NULL;
  } else if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) {
    return DR_E_ALIGN;
  }
  const bool need_write = !d->write_is_erase;
  if ((st = check_ptr(q, ex.qk, true)) || (st = check_ptr(k, ex.qk, true)) ||
      (st = check_ptr(v, ex.v, true)) || (st = check_ptr(log_decay, ex.decay, true)) ||
      (st = check_ptr(erase, ex.erase, true)) ||
      (st = check_ptr(need_write ? write : nullptr, ex.write, need_write)) ||
      (st = check_ptr(S0, ex.state, false)) || (st = check_ptr(o, ex.o, true)) ||
      (st = check_ptr(S_T, ex.state, false)) || (st = check_ptr(workspace, workspace_bytes, false)))
    return st;
  const bool work = nseq > 0 && d->T > 0;
  if (work && workspace_bytes < dr_chunk_fwd_varlen_workspace_bytes(d, nseq)) return DR_E_WORKSPACE;
  if (work && workspace == nullptr) return DR_E_WORKSPACE;

  const Range rin[] = {range_of(q, ex.qk),         range_of(k, ex.qk),
                       range_of(v, ex.v),          range_of(log_decay, ex.decay),
                       range_of(erase, ex.erase),  range_of(need_write ? write : nullptr, ex.write),
                       range_of(S0, ex.state),     range_of(cu_seqlens, cu_bytes)};
  const Range ro = range_of(o, ex.o), rs = range_of(S_T, ex.state);
  for (const Range& r : rin)
    if (overlaps(ro, r)) return DR_E_ALIAS;
  if (overlaps(ro, rs)) return DR_E_ALIAS;
  for (int i = 0; i < 8; ++i)
    if (i != 6 && overlaps(rs, rin[i])) return DR_E_ALIAS;
  if (S0 != nullptr && S_T != nullptr && S0 != S_T && overlaps(rs, rin[6])) return DR_E_ALIAS;
  const Range rw = range_of(workspace, workspace_bytes);
  for (const Range& r : rin)
    if (overlaps(rw, r)) return DR_E_ALIAS;
  if (overlaps(rw, ro) || overlaps(rw, rs)) return DR_E_ALIAS;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (nseq == 0) return DR_OK;
  if (d->T == 0) {
    if (S_T == nullptr || S_T == S0) return DR_OK;
    return launched(dr::launch_state_copy(S0, S_T, int64_t(ex.state / 4), s));
  }
  dr::Problem p = make_problem(d, q, k, v, log_decay, erase, write, S0, o, S_T);
  p.B = nseq;
  if (uses_chunk128(d)) return launched(dr::launch_chunk128_varlen(p, cu_seqlens, workspace, s));
  return launched(dr::launch_recurrent_varlen(p, cu_seqlens, workspace, s));
}

size_t dr_chunk_bwd_workspace_bytes(const dr_desc* desc) {
  Extents ex;
  if (check_desc(desc, false, &ex) != DR_OK || desc->T == 0) return 0;
  dr::Problem p = make_problem(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr);
  return uses_chunk128(desc) ? dr::bwd_chunked_workspace_bytes(p) : dr::bwd_workspace_bytes(p);
}

int dr_chunk_bwd(const dr_desc* d, const void* q, const void* k, const void* v, const float* log_decay,
                 const float* erase, const float* write, const float* S0, const float* dO,
                 const float* dS_T, float* dq, float* dk, float* dv, float* dlog_decay, float* derase,
                 float* dwrite, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_common(d, nullptr, 0, false, q, k, v, log_decay, erase, write, S0, dO, dS_T, dq, dk, dv,
                          dlog_decay, derase, dwrite, dS0, workspace, workspace_bytes, stream);
}

size_t dr_chunk_bwd_varlen_workspace_bytes(const dr_desc* desc, int32_t nseq) {
  Extents ex;
  if (check_desc(desc, false, &ex) != DR_OK || desc->B != 1 || nseq <= 0 || nseq > kMaxSeqs || desc->T == 0)
    return 0;
  dr::Problem p = make_problem(desc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr);
  p.B = nseq;
  return uses_chunk128(desc) ? dr::bwd_chunked_varlen_workspace_bytes(p) : dr::bwd_varlen_workspace_bytes(p);
}

int dr_chunk_bwd_varlen(const dr_desc* d, const int32_t* cu_seqlens, int32_t nseq, const void* q, const void* k,
                        const void* v, const float* log_decay, const float* erase, const float* write,
                        const float* S0, const float* dO, const float* dS_T, float* dq, float* dk, float* dv,
                        float* dlog_decay, float* derase, float* dwrite, float* dS0, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return chunk_bwd_common(d, cu_seqlens, nseq, true, q, k, v, log_decay, erase, write, S0, dO, dS_T, dq, dk, dv,
                          dlog_decay, derase, dwrite, dS0, workspace, workspace_bytes, stream);
}

int dr_decode_step(const dr_desc* d, const void* q, const void* k, const void* v,
                   const float* log_decay, const float* erase, const float* write, float* S,
                   void* o, void* stream) {
  Extents ex;
  int st = check_desc(d, true, &ex);
  if (st != DR_OK) return st;
  const bool need_write = !d->write_is_erase;
  if ((st = check_ptr(q, ex.qk, true)) || (st = check_ptr(k, ex.qk, true)) ||
      (st = check_ptr(v, ex.v, true)) || (st = check_ptr(log_decay, ex.decay, true)) ||
      (st = check_ptr(erase, ex.erase, true)) ||
      (st = check_ptr(need_write ? write : nullptr, ex.write, need_write)) ||
      (st = check_ptr(S, ex.state, true)) || (st = check_ptr(o, ex.o, true)))
    return st;
  const Range rin[] = {range_of(q, ex.qk),        range_of(k, ex.qk),
                       range_of(v, ex.v),         range_of(log_decay, ex.decay),
                       range_of(erase, ex.erase), range_of(need_write ? write : nullptr, ex.write)};
  const Range ro = range_of(o, ex.o), rs = range_of(S, ex.state);
  for (const Range& r : rin)
    if (overlaps(ro, r) || overlaps(rs, r)) return DR_E_ALIAS;
  if (overlaps(ro, rs)) return DR_E_ALIAS;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dr::Problem p = make_problem(d, q, k, v, log_decay, erase, write, S, o, S);
  if (d->dk == 128 && d->dv == 128) return launched(dr::launch_decode128(p, s));
  return launched(dr::launch_recurrent(p, s));
}

}  // extern "C"

namespace {

int chunk_bwd_common(const dr_desc* d, const int32_t* cu_seqlens, int32_t nseq, bool packed, const void* q,
                     const void* k, const void* v, const float* log_decay, const float* erase, const float* write,
                     const float* S0, const float* dO, const float* dS_T, float* dq, float* dk, float* dv,
                     float* dlog_decay, float* derase, float* dwrite, float* dS0, void* workspace,
                     size_t workspace_bytes, void* stream) {
  Extents ex;
  int st = check_desc(d, false, &ex);
  if (st != DR_OK) return st;
  uint64_t cu_bytes = 0;
  if (packed) {
    if (d->B != 1 || nseq < 0 || nseq > kMaxSeqs) return DR_E_SHAPE;
    const uint64_t state_elems = uint64_t(nseq) * uint64_t(d->H) * uint64_t(d->dk) * uint64_t(d->dv);
    if (state_elems > kMaxElems) return DR_E_SHAPE;
    ex.state = state_elems * 4;
    cu_bytes = (uint64_t(nseq) + 1) * 4;
    if (cu_seqlens == nullptr) {
      if (nseq > 0) return DR_E_NULL;
    } else if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) {
      return DR_E_ALIGN;
    }
  }
  const bool need_write = !d->write_is_erase;
  if (!need_write) dwrite = nullptr;
  const uint64_t bth = uint64_t(d->B) * uint64_t(d->T) * uint64_t(d->H);
  const uint64_t g_qk = bth * uint64_t(d->dk) * 4, g_v = bth * uint64_t(d->dv) * 4;
  const uint64_t g_decay = ex.decay, g_erase = ex.erase, g_write = ex.write;
  if ((st = check_ptr(q, ex.qk, true)) || (st = check_ptr(k, ex.qk, true)) ||
      (st = check_ptr(v, ex.v, true)) || (st = check_ptr(log_decay, ex.decay, true)) ||
      (st = check_ptr(erase, ex.erase, true)) ||
      (st = check_ptr(need_write ? write : nullptr, ex.write, need_write)) ||
      (st = check_ptr(S0, ex.state, false)) || (st = check_ptr(dO, g_v, true)) ||
      (st = check_ptr(dS_T, ex.state, false)) || (st = check_ptr(dq, g_qk, true)) ||
      (st = check_ptr(dk, g_qk, true)) || (st = check_ptr(dv, g_v, true)) ||
      (st = check_ptr(dlog_decay, g_decay, true)) || (st = check_ptr(derase, g_erase, true)) ||
      (st = check_ptr(dwrite, g_write, need_write)) || (st = check_ptr(dS0, ex.state, false)) ||
      (st = check_ptr(workspace, workspace_bytes, false)))
    return st;
  const bool work = d->T > 0 && (!packed || nseq > 0);
  const size_t need = !work ? 0 : packed ? dr_chunk_bwd_varlen_workspace_bytes(d, nseq) : dr_chunk_bwd_workspace_bytes(d);
  if (workspace_bytes < need) return DR_E_WORKSPACE;
  if (work && workspace == nullptr) return DR_E_WORKSPACE;

  const Range rin[] = {range_of(q, ex.qk),        range_of(k, ex.qk),         range_of(v, ex.v),
                       range_of(log_decay, ex.decay), range_of(erase, ex.erase),
                       range_of(need_write ? write : nullptr, ex.write), range_of(S0, ex.state),
                       range_of(dO, g_v),         range_of(dS_T, ex.state),   range_of(cu_seqlens, cu_bytes)};
  const Range rout[] = {range_of(dq, g_qk),         range_of(dk, g_qk),         range_of(dv, g_v),
                        range_of(dlog_decay, g_decay), range_of(derase, g_erase),
                        range_of(dwrite, g_write),  range_of(dS0, ex.state),
                        range_of(workspace, workspace_bytes)};
  const int nout = 8;
  for (int i = 0; i < nout; ++i) {
    for (const Range& r : rin)
      if (overlaps(rout[i], r)) return DR_E_ALIAS;
    for (int j2 = i + 1; j2 < nout; ++j2)
      if (overlaps(rout[i], rout[j2])) return DR_E_ALIAS;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (packed && nseq == 0) return DR_OK;
  if (d->T == 0) {
    if (dS0 == nullptr) return DR_OK;
    return launched(dr::launch_state_copy(dS_T, dS0, int64_t(ex.state / 4), s));
  }
  dr::Problem p = make_problem(d, q, k, v, log_decay, erase, write, S0, nullptr, nullptr);
  dr::BwdArgs g{dO, dS_T, dq, dk, dv, dlog_decay, derase, dwrite, dS0};
  if (packed) {
    p.B = nseq;
    if (uses_chunk128(d)) return launched(dr::launch_bwd_chunked_varlen(p, cu_seqlens, g, workspace, s));
    return launched(dr::launch_bwd_varlen(p, cu_seqlens, g, workspace, s));
  }
  if (uses_chunk128(d)) return launched(dr::launch_bwd_chunked(p, g, workspace, s));
  return launched(dr::launch_bwd(p, g, workspace, s));
}

}  // namespace
