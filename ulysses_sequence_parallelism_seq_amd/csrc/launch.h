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

int launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                         const AttnGeom& a, void* stream);
int launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, const AttnGeom& a, void* stream);

}  // namespace uly_host
