// kda_internal.h -- launch descriptors shared by the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

struct DecodeArgs {
  const void *q, *k, *v, *alpha, *beta;
  float* state;
  void* o;
  int BH, dk, dv;
  bool bf16;
  void* stream;
  // Gated DeltaNet-2 gates (both set, beta unused) or both NULL (KDA / CKDA)
  const void* erase = nullptr;  // [BH, dk]
  const void* write = nullptr;  // [BH, dv]
  // SFDA complex gates: alpha holds (Re, Im) of the gate of each key-channel pair
  bool cpx = false;
  // tokens per (b, h) in one call: inputs [B, ntok, H, .]; BH = B * H
  int ntok = 1;
  int H = 1;
};

struct ChunkArgs {
  const void *q, *k, *v, *alpha, *beta;
  const float* s0;  // may be NULL
  void* o;
  float* sT;        // may be NULL
  float* dbg;       // may be NULL (diagnostic dumps)
  int B, T, H, dk, dv;
  bool bf16;
  void* stream;
  int vt_override;  // value-tile width (64 / 128) chosen by the caller; 0 = heuristic
  // Gated DeltaNet-2 gates (both set, beta unused) or both NULL (KDA / CKDA)
  const void* erase = nullptr;  // [B, T, H, dk]
  const void* write = nullptr;  // [B, T, H, dv]
  // SFDA complex gates: alpha holds (Re, Im) of the gate of each key-channel pair
  bool cpx = false;
  // packed variable-length batch (two-pass path only): B = 1, n_seqs sequences at device
  // offsets cu[0..n_seqs]; the chunk table (gmax entries (sequence, chunk), the first
  // global chunk of each sequence, the number of chunks) lives in the workspace
  const int* cu = nullptr;
  int n_seqs = 0;
  int gmax = 0;
  const int* ctab = nullptr;       // [gmax][2]
  const int* ctab_base = nullptr;  // [n_seqs]
  const int* ctab_total = nullptr; // [1]
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_chunk(const ChunkArgs& a);
// two-pass forward: per-chunk records into ws (cpw chunks per workgroup), then the state pass
hipError_t launch_prep(const ChunkArgs& a, void* ws, int cpw);
// the same records from the bf16 kernel sized for two workgroups per compute unit
hipError_t launch_records(const ChunkArgs& a, void* ws, int cpw);
hipError_t launch_state(const ChunkArgs& a, const void* ws);
// the bf16 walk over WalkRecord records (kda_walk.hip; launch_state forwards bf16 calls)
hipError_t launch_walk(const ChunkArgs& a, const void* ws);
// Few (b, h) chains over a long sequence: the state pass splits each chain into this many
// segments (1: one walk per chain) and needs state_split_bytes of scratch after the records.
int state_segments(int B, int T, int H, int dk, int dv, bool bf16);
size_t state_split_bytes(int B, int T, int H, int dk, int dv, bool bf16);
size_t record_bytes(bool bf16, int dk);
// varlen: clamped offsets and the chunk table from a.cu (one workgroup)
hipError_t launch_varlen_table(const ChunkArgs& a, int* cs, int* ctab, int* cbase, int* ctotal);

// Backward of the chunk forward (fixed-length batches).  Gradients are fp32 in the
// layouts of their inputs; ds0 may be NULL.  ws: bwd_workspace_bytes() of scratch.
struct BwdArgs {
  const void *q, *k, *v, *alpha, *beta, *dO;
  const float* s0;   // may be NULL (zero start state)
  const float* dsT;  // may be NULL (zero final-state gradient)
  float *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
  float* ws;
  int B, T, H, Dk, Dv;
  bool bf16;
  void* stream;
  // packed variable-length batch (B = 1): the chunk table of launch_varlen_table in the
  // workspace; states are [n_seqs, H, dk, dv]; chunk blocks are laid out [H][gmax]
  const int* cs = nullptr;      // clamped offsets [n_seqs + 1]
  const int* ctab = nullptr;    // (sequence, chunk) of every global chunk [gmax][2]
  const int* cbase = nullptr;   // first global chunk of each sequence [n_seqs]
  const int* ctotal = nullptr;  // number of chunks [1]
  int n_seqs = 0, gmax = 0;
  // Gated DeltaNet-2 (beta and dbeta unused): erase gate [.., dk], write gate [.., dv] and
  // their gradients
  const void* erase = nullptr;
  const void* write = nullptr;
  float* derase = nullptr;
  float* dwrite = nullptr;
  // SFDA (complex gates in alpha's place, (Re, Im) per key-channel pair; dalpha returns
  // d/dRe, d/dIm in the same channels)
  bool cpx = false;
  // the gradient kernel's slots (grad_scratch_bytes); NULL: right after the split walks'
  // scratch of a fixed-length batch
  float* gscr = nullptr;
  int gslots = 0;
};

// fp32 offsets inside one chunk's workspace block of the backward (C = 64 rows, NB = 4
// blocks of 16): gate products, A, D, M, W, K o rho, Q o gamma (records); S_n, Delta_n
// (forward walk); dS'_n, dDelta_n (adjoint walk).
struct BwdLayout {
  int gam, rho, pin, sig, pib, A, D, M, W, KR, QG, S, DL, DS, DDL, total;
  __host__ __device__ BwdLayout(int dk, int dv) {
    const int C = 64, CK = C * dk;
    gam = 0;
    rho = gam + CK;
    pin = rho + CK;
    sig = pin + CK;
    pib = sig + CK;
    A = pib + 4 * dk;
    D = A + C * C;
    M = D + C * C;
    W = M + C * C;
    KR = W + CK;  // K o rho
    QG = KR + CK; // Q o gamma
    S = QG + CK;
    DL = S + dk * dv;
    DS = DL + C * dv;
    DDL = DS + dk * dv;
    total = (DDL + C * dv + 63) / 64 * 64;
  }
};

// The gradient kernel's own scratch, one slot per resident workgroup (fp32 offsets in a
// slot): AV, BV, dW, F [C][dk] and the anchored products PA, PD [3][C][dk].  A workgroup
// holds a slot while it runs, so the slots are rewritten chunk after chunk and the ones in
// use at once are few enough to stay in the chip's caches.  A lock word per slot follows
// the slots.
struct GradScratch {
  int AV, BV, DW, F, PA, PD, total;
  __host__ __device__ GradScratch(int dk) {
    const int CK = 64 * dk;
    AV = 0;
    BV = AV + CK;
    DW = BV + CK;
    F = DW + CK;
    PA = F + CK;
    PD = PA + 3 * CK;
    total = PD + 3 * CK;
  }
  // lock words per XCD for n slots (n / 8 of them, in whole 128-byte lines)
  __host__ __device__ static int lock_row(long n) { return (int)((n / 8 + 31) / 32 * 32); }
};
// (64 per XCD, more than the 32 gradient workgroups an XCD holds at once)
constexpr long kGradSlots = 512;
inline long grad_slots(long chunk_blocks) {  // a multiple of 8: the slots are split by XCD
  const long n = (chunk_blocks + 7) / 8 * 8;
  return n < kGradSlots ? n : kGradSlots;
}
inline size_t grad_scratch_bytes(long chunk_blocks, int dk) {
  const size_t n = (size_t)grad_slots(chunk_blocks);
  return n * GradScratch(dk).total * sizeof(float) + ((size_t)8 * GradScratch::lock_row((long)n) * 4 + 255) / 256 * 256;
}

// Few chains over long sequences: the backward walks split each chain into this many
// segments (1: one walk per chain), with bwd_split_bytes of scratch after the chunk blocks.
int bwd_walk_segments(int B, int T, int H, int dk, int dv);
size_t bwd_split_bytes(int B, int T, int H, int dk, int dv);

// chunk blocks [B H NC], the split walks' scratch, the gradient kernel's slots
inline size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv) {
  const size_t nchunks = ((size_t)T + 63) / 64;
  const size_t blocks = (size_t)B * H * nchunks;
  return blocks * BwdLayout(dk, dv).total * sizeof(float) + bwd_split_bytes(B, T, H, dk, dv) +
         grad_scratch_bytes((long)blocks, dk);
}

hipError_t launch_bwd(const BwdArgs& a);

}  // namespace kda
