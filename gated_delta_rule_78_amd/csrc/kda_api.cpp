// kda_api.cpp -- the C ABI (include/kda.h): argument checks, then one launch.
//
// All validation happens on the host before anything touches the device, so
// every error path except KDA_ERR_HIP is reachable without a GPU.
#include "../../include/kda.h"

#include <stdint.h>
#include <stdlib.h>

#include "kda_internal.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  uintptr_t a = (uintptr_t)p;
  return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool misaligned(const void* p, unsigned bytes = 16) { return ((uintptr_t)p & (bytes - 1)) != 0; }

bool supported_width(int d) { return d == 64 || d == 128; }

// KDA_VALUE_TILE=64|128 pins the chunk kernel's value-tile width (tuning aid).
int value_tile_override() {
  static const int v = [] {
    const char* e = getenv("KDA_VALUE_TILE");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// Checks common to both entry points; fills element size.
int check_shape(const kda_shape* s, bool decode, int* es) {
  if (!s) return KDA_ERR_NULL;
  if (s->dtype != KDA_BF16 && s->dtype != KDA_F32) return KDA_ERR_DTYPE;
  if (s->B < 0 || s->H < 1 || s->dk < 1 || s->dv < 1 || (!decode && s->T < 0)) return KDA_ERR_SHAPE;
  const int64_t T = decode ? 1 : s->T;
  const int64_t rows = (int64_t)s->B * T * s->H;
  if (rows > (int64_t(1) << 40) / 256) return KDA_ERR_SHAPE;
  if (!supported_width(s->dk) || !supported_width(s->dv)) return KDA_ERR_UNSUPPORTED;
  if (!decode && s->chunk != 0 && s->chunk != 64) return KDA_ERR_UNSUPPORTED;
  *es = s->dtype == KDA_BF16 ? 2 : 4;
  return KDA_OK;
}

// KDA_PREP_CPW=n pins the chunks per workgroup of the two-pass first pass (tuning aid).
int prep_cpw_override() {
  static const int v = [] {
    const char* e = getenv("KDA_PREP_CPW");
    return e ? atoi(e) : 0;
  }();
  return v;
}

size_t workspace_bytes_for(const kda_shape& s) {
  const size_t nchunks = ((size_t)s.T + 63) / 64;
  const bool bf16 = s.dtype == KDA_BF16;
  return (size_t)s.B * s.H * nchunks * kda::record_bytes(bf16, s.dk) +
         kda::state_split_bytes(s.B, s.T, s.H, s.dk, s.dv, bf16);
}

// Pointers of one chunk-forward call; the members a given entry point does not take are NULL.
struct ChunkPtrs {
  const void *q, *k, *v, *alpha, *beta;
  const float* s0;
  void* o;
  float* sT;
  float* dbg;
  void* ws;
  size_t ws_bytes;
  const void* erase = nullptr;  // Gated DeltaNet-2 gates
  const void* write = nullptr;
  bool cpx = false;             // SFDA complex gates in alpha (two-pass, bf16 only)
};

// kNeedQKAB: q, k, alpha and beta (or, with kNeedG2, the erase gate in beta's place);
// kNeedQKA: q, k and alpha only
enum : int { kNeedQKAB = 1, kNeedVO = 2, kNeedWS = 4, kNeedG2 = 8, kNeedQKA = 16 };

// Host-side checks shared by the chunk entry points (nothing touches the device).
// n_states: state tiles per head (B, or the number of sequences of a varlen batch);
// ws_need_override: workspace bytes when not the fixed-length record count.
int validate_chunk(const kda_shape* shape, const ChunkPtrs& p, int need, int64_t n_states = -1,
                   int64_t ws_need_override = -1) {
  int es = 0;
  int rc = check_shape(shape, false, &es);
  if (rc) return rc;
  const kda_shape& s = *shape;
  if (s.dtype == KDA_F32 && (s.dk != 64 || s.dv != 64)) return KDA_ERR_UNSUPPORTED;
  if (p.cpx && (s.dtype != KDA_BF16 || p.erase || p.write)) return KDA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)s.B * s.T * s.H;
  const int64_t st_bytes = (n_states < 0 ? (int64_t)s.B : n_states) * s.H * s.dk * s.dv * 4;
  const bool g2 = (need & kNeedG2) != 0;
  if (rows > 0) {
    if ((need & kNeedQKAB) && (!p.q || !p.k || !p.alpha || (g2 ? !p.erase : !p.beta))) return KDA_ERR_NULL;
    if ((need & kNeedQKA) && (!p.q || !p.k || !p.alpha)) return KDA_ERR_NULL;
    if ((need & kNeedVO) && (!p.v || !p.o || (g2 && !p.write))) return KDA_ERR_NULL;
  }
  // q, k, v, alpha, o, the gate tiles and the states move in 16-byte vectors; beta is
  // read per element
  const void* vec[] = {p.q, p.k, p.v, p.alpha, p.o, p.s0, p.sT, p.dbg, p.erase, p.write};
  for (const void* x : vec)
    if (x && misaligned(x)) return KDA_ERR_ALIGN;
  if (p.beta && misaligned(p.beta, es)) return KDA_ERR_ALIGN;
  // inputs: [0..4] and the gate tiles may not overlap any output; [5] is the start state
  const Range in[] = {range_of(p.q, p.q ? rows * s.dk * es : 0),         range_of(p.k, p.k ? rows * s.dk * es : 0),
                      range_of(p.v, p.v ? rows * s.dv * es : 0),         range_of(p.alpha, p.alpha ? rows * s.dk * es : 0),
                      range_of(p.beta, p.beta ? rows * es : 0),          range_of(p.s0, p.s0 ? st_bytes : 0),
                      range_of(p.erase, p.erase ? rows * s.dk * es : 0), range_of(p.write, p.write ? rows * s.dv * es : 0)};
  const Range ro = range_of(p.o, p.o ? rows * s.dv * es : 0);
  const Range rs = range_of(p.sT, p.sT ? st_bytes : 0);
  for (const Range& r : in)
    if (overlap(ro, r)) return KDA_ERR_ALIAS;
  for (int i = 0; i < 8; ++i)
    if (i != 5 && overlap(rs, in[i])) return KDA_ERR_ALIAS;
  if (p.s0 != p.sT && overlap(rs, in[5])) return KDA_ERR_ALIAS;  // in place is allowed
  if (overlap(rs, ro)) return KDA_ERR_ALIAS;
  if (need & kNeedWS) {
    const size_t ws_need = ws_need_override >= 0 ? (size_t)ws_need_override : workspace_bytes_for(s);
    if (ws_need > 0 && !p.ws) return KDA_ERR_NULL;
    if (p.ws_bytes < ws_need) return KDA_ERR_WORKSPACE;
    if (((uintptr_t)p.ws & 255u) != 0) return KDA_ERR_ALIGN;
    const Range rw = range_of(p.ws, (int64_t)ws_need);
    for (const Range& r : in)
      if (overlap(rw, r)) return KDA_ERR_ALIAS;
    if (overlap(rw, ro) || overlap(rw, rs)) return KDA_ERR_ALIAS;
  }
  return KDA_OK;
}

kda::ChunkArgs chunk_args(const kda_shape& s, const ChunkPtrs& p, void* stream) {
  kda::ChunkArgs a{p.q, p.k, p.v, p.alpha, p.beta, p.s0, p.o, p.sT, p.dbg, s.B, s.T, s.H, s.dk, s.dv,
                   s.dtype == KDA_BF16, stream, value_tile_override()};
  a.erase = p.erase;
  a.write = p.write;
  a.cpx = p.cpx;
  return a;
}

// pass 1 of the two-pass forward: every chunk's record, in parallel
int run_records(const kda_shape& s, const ChunkPtrs& p, void* stream) {
  const int64_t nchunks = ((int64_t)s.T + 63) / 64;
  const int64_t total = (int64_t)s.B * s.H * nchunks;
  if (total == 0) return KDA_OK;
  int cpw = prep_cpw_override();
  if (cpw <= 0) cpw = (int)((total + 1535) / 1536);  // aim at ~1.5K workgroups (6 per CU)
  if (cpw < 1) cpw = 1;
  if (cpw > nchunks) cpw = (int)nchunks;
  return kda::launch_prep(chunk_args(s, p, stream), p.ws, cpw) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// pass 2: the state walk over the records
int run_apply(const kda_shape& s, const ChunkPtrs& p, void* stream) {
  return kda::launch_state(chunk_args(s, p, stream), p.ws) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Workspace of a packed variable-length batch: records [H][gmax], then the clamped
// offsets, the chunk table, the first chunk of each sequence and the chunk count.
struct VarlenLayout {
  int64_t gmax;
  size_t off_cs, off_tab, off_base, off_total, bytes;
};

VarlenLayout varlen_layout(const kda_shape& s, int n_seqs) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  VarlenLayout L;
  L.gmax = ((int64_t)s.T + 63) / 64 + n_seqs;
  L.off_cs = up((size_t)s.H * L.gmax * kda::record_bytes(s.dtype == KDA_BF16, s.dk));
  L.off_tab = up(L.off_cs + (size_t)(n_seqs + 1) * 4);
  L.off_base = up(L.off_tab + (size_t)L.gmax * 8);
  L.off_total = up(L.off_base + (size_t)n_seqs * 4);
  L.bytes = up(L.off_total + 4);
  return L;
}

int chunk_varlen_impl(const kda_shape* shape, const int* cu, int n_seqs, ChunkPtrs p, void* stream) {
  if (!shape) return KDA_ERR_NULL;
  if (shape->B != 1 || n_seqs < 0 || n_seqs > (1 << 24)) return KDA_ERR_SHAPE;
  if (!cu) return KDA_ERR_NULL;
  if (((uintptr_t)cu & 3u) != 0) return KDA_ERR_ALIGN;
  const VarlenLayout L = varlen_layout(*shape, n_seqs);
  const bool g2 = p.erase != nullptr || p.write != nullptr;
  int rc = validate_chunk(shape, p, kNeedQKAB | kNeedVO | kNeedWS | (g2 ? kNeedG2 : 0), n_seqs, (int64_t)L.bytes);
  if (rc) return rc;
  const kda_shape& s = *shape;
  // the offsets are an input: no output (nor the workspace) may overlap them
  const Range rc_ = range_of(cu, (int64_t)(n_seqs + 1) * 4);
  const int64_t st_bytes = (int64_t)n_seqs * s.H * s.dk * s.dv * 4;
  if (overlap(rc_, range_of(p.o, (int64_t)s.T * s.H * s.dv * (s.dtype == KDA_BF16 ? 2 : 4))) ||
      overlap(rc_, range_of(p.sT, p.sT ? st_bytes : 0)) || overlap(rc_, range_of(p.ws, (int64_t)L.bytes)))
    return KDA_ERR_ALIAS;
  if (n_seqs == 0) return KDA_OK;
  char* ws = (char*)p.ws;
  kda::ChunkArgs a = chunk_args(s, p, stream);
  a.cu = (const int*)(ws + L.off_cs);  // the kernels read the clamped offsets
  a.n_seqs = n_seqs;
  a.gmax = (int)L.gmax;
  a.ctab = (const int*)(ws + L.off_tab);
  a.ctab_base = (const int*)(ws + L.off_base);
  a.ctab_total = (const int*)(ws + L.off_total);
  kda::ChunkArgs at = a;
  at.cu = cu;  // the table kernel reads the caller's offsets
  if (kda::launch_varlen_table(at, (int*)(ws + L.off_cs), (int*)(ws + L.off_tab), (int*)(ws + L.off_base),
                               (int*)(ws + L.off_total)) != hipSuccess)
    return KDA_ERR_HIP;
  const int64_t total = (int64_t)s.H * L.gmax;
  int cpw = prep_cpw_override();
  if (cpw <= 0) cpw = (int)((total + 1535) / 1536);
  if (cpw < 1) cpw = 1;
  if (cpw > L.gmax) cpw = (int)L.gmax;
  if (kda::launch_prep(a, p.ws, cpw) != hipSuccess) return KDA_ERR_HIP;
  return kda::launch_state(a, p.ws) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}


// ---- backward ---------------------------------------------------------------------

struct BwdPtrs {
  const void *q, *k, *v, *alpha, *beta;
  const float* s0;
  const void* d_o;
  const float* dsT;
  float *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
  void* ws;
  size_t ws_bytes;
  // Gated DeltaNet-2 (beta, dbeta NULL): the gates and their gradients
  const void* erase = nullptr;
  const void* write = nullptr;
  float* derase = nullptr;
  float* dwrite = nullptr;
  // SFDA: alpha / dalpha hold complex gates and their gradients, (Re, Im) per channel pair
  bool cpx = false;
};

// Workspace of a packed batch's backward: chunk blocks [H][gmax], then the chunk table
// (clamped offsets, (sequence, chunk) pairs, first chunk of each sequence, chunk count),
// then the gradient kernel's slots.
struct BwdVarlenLayout {
  int64_t gmax;
  size_t off_cs, off_tab, off_base, off_total, off_gs, bytes;
};

BwdVarlenLayout bwd_varlen_layout(const kda_shape& s, int n_seqs) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  BwdVarlenLayout L;
  L.gmax = ((int64_t)s.T + 63) / 64 + n_seqs;
  L.off_cs = up((size_t)s.H * L.gmax * kda::BwdLayout(s.dk, s.dv).total * sizeof(float));
  L.off_tab = up(L.off_cs + (size_t)(n_seqs + 1) * 4);
  L.off_base = up(L.off_tab + (size_t)L.gmax * 8);
  L.off_total = up(L.off_base + (size_t)n_seqs * 4);
  L.off_gs = up(L.off_total + 4);
  L.bytes = up(L.off_gs + kda::grad_scratch_bytes((long)s.H * L.gmax, s.dk));
  return L;
}

// n_seqs < 0: a fixed-length batch; else a packed batch of n_seqs sequences at cu
int bwd_impl(const kda_shape* shape, const int* cu, int n_seqs, const BwdPtrs& p, void* stream) {
  int es = 0;
  int rc = check_shape(shape, false, &es);
  if (rc) return rc;
  const kda_shape& s = *shape;
  const bool packed = n_seqs >= 0;
  if (packed) {
    if (s.B != 1 || n_seqs > (1 << 24)) return KDA_ERR_SHAPE;
    if (((uintptr_t)cu & 3u) != 0) return KDA_ERR_ALIGN;
  }
  const int64_t rows = (int64_t)s.B * s.T * s.H;
  const int64_t st_bytes = (int64_t)(packed ? n_seqs : s.B) * s.H * s.dk * s.dv * 4;
  const bool g2 = p.erase || p.write || p.derase || p.dwrite;
  if (rows > 0 && (!p.q || !p.k || !p.v || !p.alpha || !p.d_o || !p.dq || !p.dk || !p.dv || !p.dalpha))
    return KDA_ERR_NULL;
  if (rows > 0 && (g2 ? (!p.erase || !p.write || !p.derase || !p.dwrite) : (!p.beta || !p.dbeta)))
    return KDA_ERR_NULL;
  const BwdVarlenLayout VL = packed ? bwd_varlen_layout(s, n_seqs) : BwdVarlenLayout{};
  const size_t ws_need = packed ? VL.bytes : kda::bwd_workspace_bytes(s.B, s.T, s.H, s.dk, s.dv);
  if (ws_need > 0 && !p.ws) return KDA_ERR_NULL;
  if (p.ws_bytes < ws_need) return KDA_ERR_WORKSPACE;
  // q, k, v, alpha and d_o move in vectors; beta is read per element
  const void* in_ptrs[] = {p.q, p.k, p.v, p.alpha, p.d_o, p.erase, p.write};
  for (const void* x : in_ptrs)
    if (x && misaligned(x)) return KDA_ERR_ALIGN;
  if (p.beta && misaligned(p.beta, es)) return KDA_ERR_ALIGN;
  const void* out_ptrs[] = {p.dq, p.dk, p.dv, p.dalpha, p.ds0, p.s0, p.dsT, p.derase, p.dwrite};
  for (const void* x : out_ptrs)
    if (x && misaligned(x)) return KDA_ERR_ALIGN;
  if (p.dbeta && misaligned(p.dbeta, 4)) return KDA_ERR_ALIGN;
  if (p.ws && ((uintptr_t)p.ws & 255u) != 0) return KDA_ERR_ALIGN;
  const Range in[] = {range_of(p.q, rows * s.dk * es),       range_of(p.k, rows * s.dk * es),
                      range_of(p.v, rows * s.dv * es),       range_of(p.alpha, rows * s.dk * es),
                      range_of(p.beta, rows * es),           range_of(p.d_o, rows * s.dv * es),
                      range_of(p.s0, p.s0 ? st_bytes : 0),   range_of(p.dsT, p.dsT ? st_bytes : 0),
                      range_of(cu, packed ? (int64_t)(n_seqs + 1) * 4 : 0),
                      range_of(p.erase, p.erase ? rows * s.dk * es : 0),
                      range_of(p.write, p.write ? rows * s.dv * es : 0)};
  const Range out[] = {range_of(p.dq, rows * s.dk * 4),      range_of(p.dk, rows * s.dk * 4),
                       range_of(p.dv, rows * s.dv * 4),      range_of(p.dalpha, rows * s.dk * 4),
                       range_of(p.dbeta, p.dbeta ? rows * 4 : 0), range_of(p.ds0, p.ds0 ? st_bytes : 0),
                       range_of(p.ws, (int64_t)ws_need),
                       range_of(p.derase, p.derase ? rows * s.dk * 4 : 0),
                       range_of(p.dwrite, p.dwrite ? rows * s.dv * 4 : 0)};
  constexpr int nout = sizeof(out) / sizeof(out[0]);
  for (int i = 0; i < nout; ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r)) return KDA_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(out[i], out[j])) return KDA_ERR_ALIAS;
  }
  kda::BwdArgs a{p.q,  p.k,  p.v,      p.alpha, p.beta,           p.d_o, p.s0, p.dsT, p.dq, p.dk, p.dv, p.dalpha,
                 p.dbeta, p.ds0, (float*)p.ws, s.B, s.T, s.H, s.dk, s.dv, s.dtype == KDA_BF16, stream};
  if (g2) {
    a.erase = p.erase;
    a.write = p.write;
    a.derase = p.derase;
    a.dwrite = p.dwrite;
  }
  if (p.cpx) {
    if (g2) return KDA_ERR_UNSUPPORTED;
    a.cpx = true;
  }
  if (packed) {
    if (n_seqs == 0) return KDA_OK;
    char* ws = (char*)p.ws;
    kda::ChunkArgs t{};
    t.T = s.T;
    t.stream = stream;
    t.cu = cu;
    t.n_seqs = n_seqs;
    t.gmax = (int)VL.gmax;
    if (kda::launch_varlen_table(t, (int*)(ws + VL.off_cs), (int*)(ws + VL.off_tab), (int*)(ws + VL.off_base),
                                 (int*)(ws + VL.off_total)) != hipSuccess)
      return KDA_ERR_HIP;
    a.cs = (const int*)(ws + VL.off_cs);
    a.ctab = (const int*)(ws + VL.off_tab);
    a.cbase = (const int*)(ws + VL.off_base);
    a.ctotal = (const int*)(ws + VL.off_total);
    a.n_seqs = n_seqs;
    a.gmax = (int)VL.gmax;
    a.gscr = (float*)(ws + VL.off_gs);
  }
  return kda::launch_bwd(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "invalid shape (negative, zero or overflowing sizes)";
    case KDA_ERR_DTYPE: return "unknown dtype";
    case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KDA_ERR_ALIAS: return "an output overlaps an input it must not alias";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration (dk/dv, chunk or dtype)";
    case KDA_ERR_HIP: return "HIP runtime error on launch";
    case KDA_ERR_WORKSPACE: return "workspace smaller than kda_chunk_fwd_workspace_size()";
    case KDA_ERR_SCRATCH: return "shape needs more workspace than the fixed no-alloc scratch (KDA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int kda_version(void) { return kVersion; }


int kda_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                  const void* alpha, const void* beta, const float* initial_state, void* o,
                  float* final_state, void* stream) {
  ChunkPtrs p{q, k, v, alpha, beta, initial_state, o, final_state, nullptr, nullptr, 0};
  int rc = validate_chunk(shape, p, kNeedQKAB | kNeedVO);
  if (rc) return rc;
  if (shape->T <= 64 || (int64_t)shape->B * shape->H == 0)
    return kda::launch_chunk(chunk_args(*shape, p, stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  // more than one chunk: the two-pass forward on a workspace taken from the device's
  // stream-ordered memory pool and given back in stream order after the second pass
  const size_t need = kda_chunk_fwd_workspace_size(shape);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, need, (hipStream_t)stream) != hipSuccess || !ws) return KDA_ERR_HIP;
  p.ws = ws;
  p.ws_bytes = need;
  rc = run_records(*shape, p, stream);
  if (!rc) rc = run_apply(*shape, p, stream);
  if (hipFreeAsync(ws, (hipStream_t)stream) != hipSuccess && !rc) rc = KDA_ERR_HIP;
  return rc;
}

size_t kda_chunk_fwd_workspace_size(const kda_shape* shape) {
  int es = 0;
  if (check_shape(shape, false, &es) != KDA_OK) return 0;
  if (shape->dtype == KDA_F32 && (shape->dk != 64 || shape->dv != 64)) return 0;
  return workspace_bytes_for(*shape);
}

int kda_chunk_fwd_ws(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                     const void* beta, const float* initial_state, void* o, float* final_state, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!workspace) {  // the single-pass kernel
    const ChunkPtrs p{q, k, v, alpha, beta, initial_state, o, final_state, nullptr, nullptr, 0};
    const int rc = validate_chunk(shape, p, kNeedQKAB | kNeedVO);
    if (rc) return rc;
    return kda::launch_chunk(chunk_args(*shape, p, stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  const ChunkPtrs p{q, k, v, alpha, beta, initial_state, o, final_state, nullptr, workspace, workspace_bytes};
  int rc = validate_chunk(shape, p, kNeedQKAB | kNeedVO | kNeedWS);
  if (rc) return rc;
  rc = run_records(*shape, p, stream);
  return rc ? rc : run_apply(*shape, p, stream);
}

size_t kda_chunk_fwd_varlen_workspace_size(const kda_shape* shape, int n_seqs) {
  int es = 0;
  if (check_shape(shape, false, &es) != KDA_OK || shape->B != 1 || n_seqs < 0 || n_seqs > (1 << 24)) return 0;
  if (shape->dtype == KDA_F32 && (shape->dk != 64 || shape->dv != 64)) return 0;
  return varlen_layout(*shape, n_seqs).bytes;
}

int kda_chunk_fwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q, const void* k,
                         const void* v, const void* alpha, const void* beta, const float* initial_state, void* o,
                         float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  const ChunkPtrs p{q, k, v, alpha, beta, initial_state, o, final_state, nullptr, workspace, workspace_bytes};
  return chunk_varlen_impl(shape, cu_seqlens, n_seqs, p, stream);
}

int kda_gdn2_chunk_fwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q,
                              const void* k, const void* v, const void* alpha, const void* erase_gate,
                              const void* write_gate, const float* initial_state, void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream) {
  ChunkPtrs p{q, k, v, alpha, nullptr, initial_state, o, final_state, nullptr, workspace, workspace_bytes};
  p.erase = erase_gate;
  p.write = write_gate;
  if (!erase_gate || !write_gate) {
    if (!shape) return KDA_ERR_NULL;
    if ((int64_t)shape->T * shape->H > 0) return KDA_ERR_NULL;
  }
  return chunk_varlen_impl(shape, cu_seqlens, n_seqs, p, stream);
}

int kda_chunk_records(const kda_shape* shape, const void* q, const void* k, const void* alpha, const void* beta,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const ChunkPtrs p{q, k, nullptr, alpha, beta, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes};
  int rc = validate_chunk(shape, p, kNeedQKAB | kNeedWS);
  return rc ? rc : run_records(*shape, p, stream);
}

int kda_chunk_apply_records(const kda_shape* shape, const void* q, const void* k, const void* alpha,
                            const void* workspace, size_t workspace_bytes, const void* v,
                            const float* initial_state, void* o, float* final_state, void* stream) {
  const ChunkPtrs p{q, k, v, alpha, nullptr, initial_state, o, final_state, nullptr,
                    const_cast<void*>(workspace), workspace_bytes};
  int rc = validate_chunk(shape, p, kNeedQKA | kNeedVO | kNeedWS);
  return rc ? rc : run_apply(*shape, p, stream);
}

int kda_chunk_fwd_debug(const kda_shape* shape, const void* q, const void* k, const void* v,
                        const void* alpha, const void* beta, const float* initial_state, void* o,
                        float* final_state, float* dbg, void* stream) {
  if (!dbg) return KDA_ERR_NULL;
  const ChunkPtrs p{q, k, v, alpha, beta, initial_state, o, final_state, dbg, nullptr, 0};
  int rc = validate_chunk(shape, p, kNeedQKAB | kNeedVO);
  if (rc) return rc;
  return kda::launch_chunk(chunk_args(*shape, p, stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_gdn2_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                       const void* erase_gate, const void* write_gate, const float* initial_state, void* o,
                       float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  ChunkPtrs p{q, k, v, alpha, nullptr, initial_state, o, final_state, nullptr, workspace, workspace_bytes};
  p.erase = erase_gate;
  p.write = write_gate;
  int rc = validate_chunk(shape, p, kNeedQKAB | kNeedVO | kNeedWS | kNeedG2);
  if (rc) return rc;
  rc = run_records(*shape, p, stream);
  return rc ? rc : run_apply(*shape, p, stream);
}

// ntok < 0: the single decode step (shape->T ignored); else ntok = shape->T tokens per (b, h)
static int decode_impl(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                       const void* beta, const void* erase, const void* write, float* state, void* o,
                       void* stream, bool multi, bool cpx = false) {
  int es = 0;
  int rc = check_shape(shape, true, &es);
  if (rc) return rc;
  const kda_shape& s = *shape;
  if (multi && s.T < 0) return KDA_ERR_SHAPE;
  const int ntok = multi ? s.T : 1;
  const int64_t rows = (int64_t)s.B * s.H;             // states
  const int64_t trows = rows * ntok;                    // token rows of the inputs and o
  if (rows > 0x7FFFFFFF || trows > (int64_t(1) << 40) / 256) return KDA_ERR_SHAPE;
  const bool g2 = erase || write;
  if (trows > 0 && (!q || !k || !v || !alpha || !o || !state || (g2 ? (!erase || !write) : !beta)))
    return KDA_ERR_NULL;
  // the state moves in 16-byte vectors; the per-token vectors are read per element
  if (state && misaligned(state)) return KDA_ERR_ALIGN;
  const void* ptrs[] = {q, k, v, alpha, beta, o, erase, write};
  for (const void* p : ptrs)
    if (p && misaligned(p, es)) return KDA_ERR_ALIGN;
  const Range in[] = {range_of(q, trows * s.dk * es),     range_of(k, trows * s.dk * es),
                      range_of(v, trows * s.dv * es),     range_of(alpha, trows * s.dk * es),
                      range_of(beta, beta ? trows * es : 0), range_of(erase, erase ? trows * s.dk * es : 0),
                      range_of(write, write ? trows * s.dv * es : 0)};
  const Range ro = range_of(o, trows * s.dv * es);
  const Range rs = range_of(state, rows * s.dk * s.dv * 4);
  for (const Range& r : in)
    if (overlap(ro, r) || overlap(rs, r)) return KDA_ERR_ALIAS;
  if (overlap(ro, rs)) return KDA_ERR_ALIAS;
  if (ntok == 0) return KDA_OK;
  kda::DecodeArgs a{q, k, v, alpha, beta, state, o, (int)rows, s.dk, s.dv, s.dtype == KDA_BF16, stream};
  a.erase = erase;
  a.write = write;
  a.ntok = ntok;
  a.H = s.H;
  a.cpx = cpx;
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_gdn2_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                         const void* erase_gate, const void* write_gate, float* state, void* o, void* stream) {
  if (!erase_gate || !write_gate) {
    int es = 0;
    int rc = check_shape(shape, true, &es);
    if (rc) return rc;
    if ((int64_t)shape->B * shape->H > 0) return KDA_ERR_NULL;
  }
  return decode_impl(shape, q, k, v, alpha, nullptr, erase_gate, write_gate, state, o, stream, false);
}

int kda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                    const void* alpha, const void* beta, float* state, void* o, void* stream) {
  return decode_impl(shape, q, k, v, alpha, beta, nullptr, nullptr, state, o, stream, false);
}

int kda_decode_tokens(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                      const void* beta, float* state, void* o, void* stream) {
  return decode_impl(shape, q, k, v, alpha, beta, nullptr, nullptr, state, o, stream, true);
}

int kda_gdn2_decode_tokens(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                           const void* erase_gate, const void* write_gate, float* state, void* o, void* stream) {
  if (!erase_gate || !write_gate) {
    int es = 0;
    int rc = check_shape(shape, true, &es);
    if (rc) return rc;
    if ((int64_t)shape->B * shape->H > 0) return KDA_ERR_NULL;
  }
  return decode_impl(shape, q, k, v, alpha, nullptr, erase_gate, write_gate, state, o, stream, true);
}

int kda_sfda_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v, const void* lambda,
                       const void* beta, const float* initial_state, void* o, float* final_state, void* workspace,
                       size_t workspace_bytes, void* stream) {
  ChunkPtrs p{q, k, v, lambda, beta, initial_state, o, final_state, nullptr, workspace, workspace_bytes};
  p.cpx = true;
  int rc = validate_chunk(shape, p, kNeedQKAB | kNeedVO | kNeedWS);
  if (rc) return rc;
  rc = run_records(*shape, p, stream);
  return rc ? rc : run_apply(*shape, p, stream);
}

int kda_sfda_chunk_fwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q,
                              const void* k, const void* v, const void* lambda, const void* beta,
                              const float* initial_state, void* o, float* final_state, void* workspace,
                              size_t workspace_bytes, void* stream) {
  ChunkPtrs p{q, k, v, lambda, beta, initial_state, o, final_state, nullptr, workspace, workspace_bytes};
  p.cpx = true;
  return chunk_varlen_impl(shape, cu_seqlens, n_seqs, p, stream);
}

int kda_sfda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v, const void* lambda,
                         const void* beta, float* state, void* o, void* stream) {
  return decode_impl(shape, q, k, v, lambda, beta, nullptr, nullptr, state, o, stream, false, true);
}

int kda_sfda_decode_tokens(const kda_shape* shape, const void* q, const void* k, const void* v, const void* lambda,
                           const void* beta, float* state, void* o, void* stream) {
  return decode_impl(shape, q, k, v, lambda, beta, nullptr, nullptr, state, o, stream, true, true);
}

size_t kda_chunk_bwd_workspace_size(const kda_shape* shape) {
  int es = 0;
  if (check_shape(shape, false, &es) != KDA_OK) return 0;
  return kda::bwd_workspace_bytes(shape->B, shape->T, shape->H, shape->dk, shape->dv);
}

int kda_chunk_bwd(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                  const void* beta, const float* initial_state, const void* d_o, const float* d_final_state,
                  float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* d_initial_state,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const BwdPtrs p{q, k, v, alpha, beta, initial_state, d_o, d_final_state, dq, dk, dv, dalpha, dbeta, d_initial_state,
                  workspace, workspace_bytes};
  return bwd_impl(shape, nullptr, -1, p, stream);
}

size_t kda_chunk_bwd_varlen_workspace_size(const kda_shape* shape, int n_seqs) {
  int es = 0;
  if (check_shape(shape, false, &es) != KDA_OK || shape->B != 1 || n_seqs < 0 || n_seqs > (1 << 24)) return 0;
  return bwd_varlen_layout(*shape, n_seqs).bytes;
}

int kda_chunk_bwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q, const void* k,
                         const void* v, const void* alpha, const void* beta, const float* initial_state,
                         const void* d_o, const float* d_final_state, float* dq, float* dk, float* dv,
                         float* dalpha, float* dbeta, float* d_initial_state, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!shape) return KDA_ERR_NULL;
  if (n_seqs < 0) return KDA_ERR_SHAPE;
  if (!cu_seqlens) return KDA_ERR_NULL;
  const BwdPtrs p{q, k, v, alpha, beta, initial_state, d_o, d_final_state, dq, dk, dv, dalpha, dbeta, d_initial_state,
                  workspace, workspace_bytes};
  return bwd_impl(shape, cu_seqlens, n_seqs, p, stream);
}

int kda_gdn2_chunk_bwd(const kda_shape* shape, const void* q, const void* k, const void* v, const void* alpha,
                       const void* erase_gate, const void* write_gate, const float* initial_state, const void* d_o,
                       const float* d_final_state, float* dq, float* dk, float* dv, float* dalpha, float* d_erase,
                       float* d_write, float* d_initial_state, void* workspace, size_t workspace_bytes,
                       void* stream) {
  BwdPtrs p{q, k, v, alpha, nullptr, initial_state, d_o, d_final_state, dq, dk, dv, dalpha, nullptr, d_initial_state,
            workspace, workspace_bytes};
  p.erase = erase_gate;
  p.write = write_gate;
  p.derase = d_erase;
  p.dwrite = d_write;
  if (!erase_gate || !write_gate || !d_erase || !d_write) {
    if (!shape) return KDA_ERR_NULL;
    if ((int64_t)shape->B * shape->T * shape->H > 0) return KDA_ERR_NULL;
  }
  return bwd_impl(shape, nullptr, -1, p, stream);
}

int kda_gdn2_chunk_bwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q,
                              const void* k, const void* v, const void* alpha, const void* erase_gate,
                              const void* write_gate, const float* initial_state, const void* d_o,
                              const float* d_final_state, float* dq, float* dk, float* dv, float* dalpha,
                              float* d_erase, float* d_write, float* d_initial_state, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!shape) return KDA_ERR_NULL;
  if (n_seqs < 0) return KDA_ERR_SHAPE;
  if (!cu_seqlens) return KDA_ERR_NULL;
  BwdPtrs p{q, k, v, alpha, nullptr, initial_state, d_o, d_final_state, dq, dk, dv, dalpha, nullptr, d_initial_state,
            workspace, workspace_bytes};
  p.erase = erase_gate;
  p.write = write_gate;
  p.derase = d_erase;
  p.dwrite = d_write;
  if (!erase_gate || !write_gate || !d_erase || !d_write) {
    if ((int64_t)shape->T * shape->H > 0) return KDA_ERR_NULL;
  }
  return bwd_impl(shape, cu_seqlens, n_seqs, p, stream);
}

int kda_sfda_chunk_bwd(const kda_shape* shape, const void* q, const void* k, const void* v, const void* lambda,
                       const void* beta, const float* initial_state, const void* d_o, const float* d_final_state,
                       float* dq, float* dk, float* dv, float* dlambda, float* dbeta, float* d_initial_state,
                       void* workspace, size_t workspace_bytes, void* stream) {
  BwdPtrs p{q, k, v, lambda, beta, initial_state, d_o, d_final_state, dq, dk, dv, dlambda, dbeta, d_initial_state,
            workspace, workspace_bytes};
  p.cpx = true;
  return bwd_impl(shape, nullptr, -1, p, stream);
}

int kda_sfda_chunk_bwd_varlen(const kda_shape* shape, const int* cu_seqlens, int n_seqs, const void* q,
                              const void* k, const void* v, const void* lambda, const void* beta,
                              const float* initial_state, const void* d_o, const float* d_final_state, float* dq,
                              float* dk, float* dv, float* dlambda, float* dbeta, float* d_initial_state,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape) return KDA_ERR_NULL;
  if (n_seqs < 0) return KDA_ERR_SHAPE;
  if (!cu_seqlens) return KDA_ERR_NULL;
  BwdPtrs p{q, k, v, lambda, beta, initial_state, d_o, d_final_state, dq, dk, dv, dlambda, dbeta, d_initial_state,
            workspace, workspace_bytes};
  p.cpx = true;
  return bwd_impl(shape, cu_seqlens, n_seqs, p, stream);
}

}  // extern "C"
