// Internal launchers shared between the translation units of the library.
#pragma once

#include <stddef.h>

namespace uly_host {

// Geometry of one attention call: G = sp * B independent rows of N tokens,
// Hl heads of width d; token t of (row g, head h) starts at element
// ((g * N + t) * Hl + h) * d.
struct AttnGeom {
  int G, N, Hl, d;
  const int* cu;  // device int32 [ndoc + 1] or nullptr
  int ndoc;       // 1 when cu == nullptr
  int max_doc_len;
  int causal;
};

int launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                        const AttnGeom& a, void* stream);
int launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                        const float* dout, const float* lse, float* dq, float* dk, float* dv,
                        float* delta, const AttnGeom& a, void* stream);
// The backward's two steps: the D pre-pass into the workspace, then the
// dQ and dK/dV kernels reading it.
int launch_attn_bwd_prepare_f32(const float* o, const float* dout, float* delta, const AttnGeom& a,
                                void* stream);
int launch_attn_bwd_main_f32(const float* q, const float* k, const float* v, const float* dout,
                             const float* lse, float* dq, float* dk, float* dv, const float* delta,
                             const AttnGeom& a, void* stream);

// sched: kQueueInts ints of caller memory for a persistent launch, or nullptr
int launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                         const AttnGeom& a, void* stream, int* sched);
int launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, const AttnGeom& a, void* stream);
// with_sched: the workspace also holds the persistent kernels' queue
// counters (ulysses_attn_bwd's layout), which the pre-pass clears.
int launch_attn_bwd_prepare_bf16(const void* o, const void* dout, const float* lse, float* delta,
                                 const AttnGeom& a, void* stream, bool with_sched);
int launch_attn_bwd_main_bf16(const void* q, const void* k, const void* v, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, const float* delta,
                              const AttnGeom& a, void* stream);

// Ring attention steps (bf16): rows g = chunk * B + b of Ns tokens, H heads.
// sched: the forward's queue counters (ulysses_attn_fwd_workspace_bytes) for
// a persistent launch, or nullptr for one workgroup per tile.
int launch_ring_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* o_acc, float* lse,
                         const AttnGeom& a, int sp, int B, int step, void* stream, int* sched);
// delta: the workspace the ring prepare call filled (ring_bwd_workspace_bytes
// of it), whose queue counters the step's persistent kernels claim from.
int launch_ring_bwd_bf16(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                         float* delta, float* dq_acc, float* dk_acc, float* dv_acc, void* dq, void* dk,
                         void* dv, const AttnGeom& a, int sp, int B, int step, void* stream);
// Bytes of a backward workspace over `rows` (rank, batch row, head, token)
// rows: -D and lse in log2 units, then the two kernels' queue counters.
size_t bwd_workspace_bytes(size_t rows);

}  // namespace uly_host
