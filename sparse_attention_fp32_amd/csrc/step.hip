// One decode step from one host call: the fused calls in pipeline order
// (Atlas glm5next_dsa page, "Shape of the pipeline": compression, index
// scores, top-k, expansion, sparse MLA; the head-gate of stkernel pull request
// #227 rides in the compression launch).
//
// The step makes the same calls a caller would make one by one, so its results
// are theirs bit for bit.  What it changes is the host side: one call per step
// instead of four or five, which lets one host thread keep the stream's queue
// ahead of the kernels without capturing a graph.  Every call is first run as
// a dry run (argument checks only, nothing launched), so a bad argument of the
// last call returns before the first one is enqueued.
#include "dsa_host.hpp"

namespace {

dsa_status run_calls(const dsa_decode_step_args* a, hipStream_t stream) {
  dsa_status st = dsa_gate_compress(
      a->hidden, a->W, a->M, a->K, a->H, a->gate_part, a->gate_part_bytes, a->k, a->gate, a->ape,
      a->valid, a->tok_off, a->pool_off, a->seq_len, a->ln_w, a->ln_b, a->eps, a->B, a->D,
      a->kpool, a->max_cap, a->new_from, a->max_new, a->keys, a->pool_start, a->pool_valid,
      a->n_pools, stream);
  if (st != DSA_OK) return st;
  const int nslices = dsa_gate_split_count(a->M, a->K, a->H);
  DSA_REQUIRE(nslices >= 1, DSA_ERR_INVALID_ARG, "dsa_decode_step: no head-gate split for M=%d K=%d H=%d",
              a->M, a->K, a->H);
  st = dsa_index_scores_gated(a->qi, a->gate_part, nslices, a->w, a->keys, a->pool_start,
                              a->pool_valid, a->pool_off, a->n_pools, a->q_req, a->q_pos, a->Q,
                              a->H, a->D, a->kpool, a->pstride, a->scores, a->cand, stream);
  if (st != DSA_OK) return st;
  st = dsa_topk_expand(a->scores, a->cand, a->row_len, a->Q, a->pstride, a->select_k,
                       a->pool_start, a->pool_off, a->q_req, a->kpool, a->out_width,
                       a->topk_flags, a->sel, a->tok, stream);
  if (st != DSA_OK) return st;
  if (a->select_tail) {
    st = dsa_select_tail(a->valid, a->tok_off, a->pool_start, a->pool_off, a->n_pools, a->q_req,
                         a->q_pos, a->Q, a->kpool, a->select_k, a->out_width, a->tok, stream);
    if (st != DSA_OK) return st;
  }
  if (a->block_table)
    return dsa_sparse_mla_decode_paged(a->q_mla, a->ckv, a->ckv_scale, a->latent_dtype,
                                       a->block_table, a->bt_stride, a->page_rows, a->n_pages,
                                       a->q_req, a->tok, a->Q, a->Hm, a->L, a->out_width,
                                       a->sm_scale, a->out, a->lse, a->kvidx, a->mla_ws,
                                       a->mla_ws_bytes, stream);
  return dsa_sparse_mla_decode(a->q_mla, a->ckv, a->ckv_scale, a->latent_dtype, a->kv_off,
                               a->q_req, a->tok, a->Q, a->Hm, a->L, a->out_width, a->sm_scale,
                               a->out, a->lse, a->mla_ws, a->mla_ws_bytes, stream);
}

}  // namespace

DSA_EXPORT size_t dsa_decode_step_args_size(void) { return sizeof(dsa_decode_step_args); }

DSA_EXPORT dsa_status dsa_decode_step(const dsa_decode_step_args* a, hipStream_t stream) {
  DSA_REQUIRE(a, DSA_ERR_INVALID_ARG, "dsa_decode_step: NULL argument block");
  DSA_REQUIRE(a->struct_bytes == sizeof(dsa_decode_step_args), DSA_ERR_INVALID_ARG,
              "dsa_decode_step: struct_bytes=%zu, the library's layout has %zu", a->struct_bytes,
              sizeof(dsa_decode_step_args));
  DSA_REQUIRE(a->M == a->Q, DSA_ERR_INVALID_ARG,
              "dsa_decode_step: the head-gate rows M=%d must be the step's queries Q=%d", a->M,
              a->Q);
  {
    const dsa::DryRun dry;
    const dsa_status st = run_calls(a, stream);
    if (st != DSA_OK) return st;
  }
  return run_calls(a, stream);
}
