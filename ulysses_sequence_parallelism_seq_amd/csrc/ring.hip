// Entry points of ring attention, the other sequence-parallel mode the
// ColossalAI docs ("Sequence Parallelism") offer beside Ulysses
// (sequence_parallelism_mode="ring_attn"; related paper: Ring Attention with
// Blockwise Transformers), for sp virtual ranks held on one device.
//
// Rank r keeps token chunk r of q, k, v for all heads, [sp][B][Ns][H][d]. At
// ring step i it holds key/value chunk j = (r - i) mod sp and attends its
// queries to that block (causal: j < r the whole chunk, j == r the causal
// diagonal, j > r nothing), merging the block's partial result with its
// running one by log-sum-exp. The forward kernel does the merge in place: it
// resumes the online softmax from the running (O, lse) (see attn_fwd.hip).
// The backward, given the final lse and D = rowsum(dO * O), adds each block's
// terms to fp32 running sums: dQ of the query chunk, dK and dV of the
// key/value chunk (which travel with the chunk on a real ring).
//
// The kernels are the Ulysses attention kernels in ring mode: the stacked
// rows g = chunk * B + b of Ns tokens take the place of the G = sp * B rows
// of N tokens, the H heads that of the Hl local heads.

#include "common.h"
#include "launch.h"

namespace {

int check_ring(int step, int sp, int B, int Ns, int H, int d, int dtype) {
  const int rc = uly_host::check_attn_args(1, Ns, nullptr, sp, B, Ns, H, d, dtype);
  if (rc != ULY_OK) return rc;
  if (dtype != ULY_BF16) return ULY_EUNSUPPORTED;
  if (step < 0 || step >= sp) return ULY_EINVAL;
  return ULY_OK;
}

uly_host::AttnGeom ring_geom(int sp, int B, int Ns, int H, int d, int causal) {
  uly_host::AttnGeom g;
  g.G = sp * B;
  g.N = Ns;
  g.Hl = H;
  g.d = d;
  g.cu = nullptr;
  g.ndoc = 1;
  g.max_doc_len = Ns;
  g.causal = causal ? 1 : 0;
  return g;
}

}  // namespace

extern "C" int ulysses_ring_attn_fwd_step(const void* q, const void* k, const void* v, void* o, float* o_acc,
                                          float* lse, int step, int sp, int B, int Ns, int H, int d, int causal,
                                          int dtype, void* stream) {
  if (!q || !k || !v || !o || !o_acc || !lse) return ULY_EINVAL;
  const int rc = check_ring(step, sp, B, Ns, H, d, dtype);
  if (rc != ULY_OK) return rc;
  return uly_host::launch_ring_fwd_bf16(q, k, v, o, o_acc, lse, ring_geom(sp, B, Ns, H, d, causal), sp, B, step,
                                        stream, nullptr);
}

extern "C" int ulysses_ring_attn_fwd_step_ws(const void* q, const void* k, const void* v, void* o, float* o_acc,
                                             float* lse, void* workspace, size_t workspace_bytes, int step, int sp,
                                             int B, int Ns, int H, int d, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !o_acc || !lse) return ULY_EINVAL;
  const int rc = check_ring(step, sp, B, Ns, H, d, dtype);
  if (rc != ULY_OK) return rc;
  if (!workspace || workspace_bytes < ulysses_attn_fwd_workspace_bytes()) return ULY_EWORKSPACE;
  return uly_host::launch_ring_fwd_bf16(q, k, v, o, o_acc, lse, ring_geom(sp, B, Ns, H, d, causal), sp, B, step,
                                        stream, static_cast<int*>(workspace));
}

extern "C" size_t ulysses_ring_attn_bwd_workspace_bytes(int sp, int B, int Ns, int H, int d, int dtype) {
  if (check_ring(0, sp, B, Ns, H, d, dtype) != ULY_OK) return 0;
  // -D and lse in log2 units: two floats per (rank, batch row, head, token),
  // then the queue counters of the steps' persistent kernels
  return uly_host::bwd_workspace_bytes((size_t)sp * B * H * Ns);
}

extern "C" int ulysses_ring_attn_bwd_prepare(const void* o, const void* dout, const float* lse, void* workspace,
                                             size_t workspace_bytes, int sp, int B, int Ns, int H, int d,
                                             int dtype, void* stream) {
  if (!o || !dout || !lse) return ULY_EINVAL;
  const int rc = check_ring(0, sp, B, Ns, H, d, dtype);
  if (rc != ULY_OK) return rc;
  if (!workspace || workspace_bytes < ulysses_ring_attn_bwd_workspace_bytes(sp, B, Ns, H, d, dtype))
    return ULY_EWORKSPACE;
  return uly_host::launch_attn_bwd_prepare_bf16(o, dout, lse, static_cast<float*>(workspace),
                                                ring_geom(sp, B, Ns, H, d, 1), stream, true);
}

extern "C" int ulysses_ring_attn_bwd_step(const void* q, const void* k, const void* v, const void* dout,
                                          const float* lse, void* workspace, size_t workspace_bytes,
                                          float* dq_acc, float* dk_acc, float* dv_acc, void* dq, void* dk, void* dv,
                                          int step, int sp, int B, int Ns, int H, int d, int causal, int dtype,
                                          void* stream) {
  if (!q || !k || !v || !dout || !lse || !dq_acc || !dk_acc || !dv_acc || !dq || !dk || !dv) return ULY_EINVAL;
  const int rc = check_ring(step, sp, B, Ns, H, d, dtype);
  if (rc != ULY_OK) return rc;
  if (!workspace || workspace_bytes < ulysses_ring_attn_bwd_workspace_bytes(sp, B, Ns, H, d, dtype))
    return ULY_EWORKSPACE;
  return uly_host::launch_ring_bwd_bf16(q, k, v, dout, lse, static_cast<float*>(workspace), dq_acc, dk_acc,
                                        dv_acc, dq, dk, dv, ring_geom(sp, B, Ns, H, d, causal), sp, B, step,
                                        stream);
}
