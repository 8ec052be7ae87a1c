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
    default: return "unknown status";
  }
}

int kda_version(void) { return kVersion; }

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
  return (size_t)s.B * s.H * nchunks * kda::record_bytes(s.dtype == KDA_BF16, s.dk);
}

static int chunk_fwd_impl(const kda_shape* shape, const void* q, const void* k, const void* v,
                          const void* alpha, const void* beta, const float* s0, void* o, float* sT,
                          float* dbg, void* ws, size_t ws_bytes, void* stream) {
  int es = 0;
  int rc = check_shape(shape, false, &es);
  if (rc) return rc;
  const kda_shape& s = *shape;
  if (s.dtype == KDA_F32 && (s.dk != 64 || s.dv != 64)) return KDA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)s.B * s.T * s.H;
  const int64_t st_bytes = (int64_t)s.B * s.H * s.dk * s.dv * 4;
  if (rows > 0 && (!q || !k || !v || !alpha || !beta || !o)) return KDA_ERR_NULL;
  // q, k, v, alpha, o and the states move in 16-byte vectors; beta is read per element
  const void* ptrs[] = {q, k, v, alpha, o, s0, sT, dbg};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return KDA_ERR_ALIGN;
  if (beta && misaligned(beta, es)) return KDA_ERR_ALIGN;
  const Range in[] = {range_of(q, rows * s.dk * es), range_of(k, rows * s.dk * es),
                      range_of(v, rows * s.dv * es), range_of(alpha, rows * s.dk * es),
                      range_of(beta, rows * es), range_of(s0, s0 ? st_bytes : 0)};
  const Range ro = range_of(o, rows * s.dv * es);
  for (const Range& r : in)
    if (overlap(ro, r)) return KDA_ERR_ALIAS;
  if (sT) {
    const Range rs = range_of(sT, st_bytes);
    for (int i = 0; i < 5; ++i)
      if (overlap(rs, in[i])) return KDA_ERR_ALIAS;
    if (s0 && s0 != sT && overlap(rs, in[5])) return KDA_ERR_ALIAS;
    if (overlap(rs, ro)) return KDA_ERR_ALIAS;
  }
  kda::ChunkArgs a{q, k, v, alpha, beta, s0, o, sT, dbg, s.B, s.T, s.H, s.dk, s.dv,
                   s.dtype == KDA_BF16, stream, value_tile_override()};
  if (!ws) return kda::launch_chunk(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  // two-pass path: the workspace holds one record per (b, h, chunk)
  const size_t need = workspace_bytes_for(s);
  if (ws_bytes < need) return KDA_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return KDA_ERR_ALIGN;
  const Range rw = range_of(ws, (int64_t)need);
  for (const Range& r : in)
    if (overlap(rw, r)) return KDA_ERR_ALIAS;
  if (overlap(rw, ro) || (sT && overlap(rw, range_of(sT, st_bytes)))) return KDA_ERR_ALIAS;
  if (rows == 0) return kda::launch_state(a, ws) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  const int64_t nchunks = ((int64_t)s.T + 63) / 64;
  const int64_t total = (int64_t)s.B * s.H * nchunks;
  int cpw = prep_cpw_override();
  if (cpw <= 0) cpw = (int)((total + 1535) / 1536);  // aim at ~1.5K workgroups (6 per CU)
  if (cpw < 1) cpw = 1;
  if (cpw > nchunks) cpw = (int)nchunks;
  if (kda::launch_prep(a, ws, cpw) != hipSuccess) return KDA_ERR_HIP;
  return kda::launch_state(a, ws) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                  const void* alpha, const void* beta, const float* initial_state, void* o,
                  float* final_state, void* stream) {
  return chunk_fwd_impl(shape, q, k, v, alpha, beta, initial_state, o, final_state, nullptr, nullptr, 0, stream);
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
  return chunk_fwd_impl(shape, q, k, v, alpha, beta, initial_state, o, final_state, nullptr, workspace,
                        workspace_bytes, stream);
}

int kda_chunk_fwd_debug(const kda_shape* shape, const void* q, const void* k, const void* v,
                        const void* alpha, const void* beta, const float* initial_state, void* o,
                        float* final_state, float* dbg, void* stream) {
  if (!dbg) return KDA_ERR_NULL;
  return chunk_fwd_impl(shape, q, k, v, alpha, beta, initial_state, o, final_state, dbg, nullptr, 0, stream);
}

int kda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                    const void* alpha, const void* beta, float* state, void* o, void* stream) {
  int es = 0;
  int rc = check_shape(shape, true, &es);
  if (rc) return rc;
  const kda_shape& s = *shape;
  const int64_t rows = (int64_t)s.B * s.H;
  if (rows > 0x7FFFFFFF) return KDA_ERR_SHAPE;
  if (rows > 0 && (!q || !k || !v || !alpha || !beta || !o || !state)) return KDA_ERR_NULL;
  // the state moves in 16-byte vectors; the per-token vectors are read per element
  if (state && misaligned(state)) return KDA_ERR_ALIGN;
  const void* ptrs[] = {q, k, v, alpha, beta, o};
  for (const void* p : ptrs)
    if (p && misaligned(p, es)) return KDA_ERR_ALIGN;
  const Range in[] = {range_of(q, rows * s.dk * es), range_of(k, rows * s.dk * es),
                      range_of(v, rows * s.dv * es), range_of(alpha, rows * s.dk * es),
                      range_of(beta, rows * es)};
  const Range ro = range_of(o, rows * s.dv * es);
  const Range rs = range_of(state, rows * s.dk * s.dv * 4);
  for (const Range& r : in)
    if (overlap(ro, r) || overlap(rs, r)) return KDA_ERR_ALIAS;
  if (overlap(ro, rs)) return KDA_ERR_ALIAS;
  kda::DecodeArgs a{q, k, v, alpha, beta, state, o, (int)rows, s.dk, s.dv, s.dtype == KDA_BF16, stream};
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
