// The cache-write side of a decode step: the step's geometry derived on the
// device from the live lengths, and the store of the step's indexer row at a
// device-side position.
//
// Atlas glm5next_dsa page, the Glm5NextDsaKernels list: write_geom derives the
// selector geometry from seq_len on the device so that a captured graph
// replays over the live context rather than the one it was captured with;
// indexer_store puts the staged indexer row at a position held in device
// memory and marks the row valid (the host-side row offset it replaces froze
// the position into the graph).  The page's k_normed buffer holds that row per
// token; with a LayerNorm the store writes k_norm of the staged row (the
// per-token reading), without one the raw row (the pooled-then-normalised
// reading of the pipeline diagram).
//
// Both are a few hundred bytes per request: one dependent load chain, no
// reuse, latency-bound.
#include <limits.h>

#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

// One thread per request.
__global__ __launch_bounds__(256) void write_geom_kernel(
    const int32_t* __restrict__ seq_len, int B, const int32_t* __restrict__ block_table,
    int bt_stride, int page_rows, int n_pages, int32_t* __restrict__ q_req,
    int32_t* __restrict__ q_pos, int32_t* __restrict__ new_from, int32_t* __restrict__ slot) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= B) return;
  const int n = max(seq_len[r], 0);
  if (q_req) q_req[r] = r;
  q_pos[r] = n - 1;
  if (new_from) new_from[r] = max(n - 1, 0);
  if (slot) {
    // the page of the newest row; block and page numbers clamped as the paged
    // attention clamps them
    const unsigned x = (unsigned)max(n - 1, 0), pr = (unsigned)page_rows;
    const unsigned b = min(x / pr, (unsigned)bt_stride - 1);
    const unsigned pg =
        min((unsigned)block_table[(int64_t)r * bt_stride + b], (unsigned)n_pages - 1);
    slot[r] = n > 0 ? (int)(pg * pr + x % pr) : -1;
  }
}

// D/8 lanes per request, 8 channels per lane (one 16-byte load per row).
template <int LPP>
__global__ __launch_bounds__(256) void indexer_store_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ gate_new,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ tok_off,
    const float* __restrict__ ln_w, const float* __restrict__ ln_b, float eps, int B,
    uint16_t* __restrict__ k, uint16_t* __restrict__ gate, uint8_t* __restrict__ valid) {
  constexpr int D = LPP * 8;
  const int t = threadIdx.x;
  const int r = blockIdx.x * (256 / LPP) + t / LPP;
  const int li = t % LPP, c0 = li * 8;
  if (r >= B) return;  // whole lane groups leave together
  const uint4 kv = *(const uint4*)(k_new + (int64_t)r * D + c0);
  const uint4 gv = *(const uint4*)(gate_new + (int64_t)r * D + c0);
  const int p = pos[r];
  const int64_t row0 = tok_off[r];
  const int region = tok_off[r + 1] - (int)row0;
  uint4 out = kv;
  if (ln_w) {
    float x[8], lw[8], lb[8];
    bf16x8_to_f32(kv, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      lw[c] = ln_w[c0 + c];
      lb[c] = ln_b[c0 + c];
    }
    out = layer_norm8_bf16<LPP>(x, lw, lb, eps);
  }
  if (p < 0 || p >= region) return;  // outside the request's region: nothing stored
  const int64_t row = row0 + p;
  *(uint4*)(k + row * D + c0) = out;
  *(uint4*)(gate + row * D + c0) = gv;
  if (li == 0) valid[row] = 1;
}

}  // namespace

DSA_EXPORT dsa_status dsa_write_geom(const int32_t* seq_len, int B, const int32_t* block_table,
                                     int bt_stride, int page_rows, int n_pages, int32_t* q_req,
                                     int32_t* q_pos, int32_t* new_from, int32_t* slot,
                                     hipStream_t stream) {
  DSA_REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "dsa_write_geom: B=%d < 0", B);
  if (slot)
    DSA_REQUIRE(block_table && bt_stride >= 1 && page_rows >= 1 && n_pages >= 1 &&
                    (long long)n_pages * page_rows <= INT_MAX,
                DSA_ERR_INVALID_ARG,
                "dsa_write_geom: slot needs a block table (bt_stride=%d, page_rows=%d, "
                "n_pages=%d)",
                bt_stride, page_rows, n_pages);
  if (B == 0) return DSA_OK;
  DSA_REQUIRE(seq_len && q_pos, DSA_ERR_INVALID_ARG, "dsa_write_geom: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_write_geom", seq_len, block_table, q_req, q_pos, new_from, slot);
  if (dsa::dry_run()) return DSA_OK;
  write_geom_kernel<<<(B + 255) / 256, 256, 0, stream>>>(seq_len, B, block_table, bt_stride,
                                                          page_rows, n_pages, q_req, q_pos,
                                                          new_from, slot);
  return dsa::check_launch("dsa_write_geom");
}

DSA_EXPORT dsa_status dsa_indexer_store(const uint16_t* k_new, const uint16_t* gate_new,
                                        const int32_t* pos, const int32_t* tok_off,
                                        const float* ln_w, const float* ln_b, float eps, int B,
                                        int D, uint16_t* k, uint16_t* gate, uint8_t* valid,
                                        hipStream_t stream) {
  DSA_REQUIRE(B >= 0, DSA_ERR_INVALID_ARG, "dsa_indexer_store: B=%d < 0", B);
  DSA_REQUIRE(D == 32 || D == 64 || D == 128 || D == 256, DSA_ERR_UNSUPPORTED,
              "dsa_indexer_store: D=%d not in {32,64,128,256}", D);
  DSA_REQUIRE((ln_w == nullptr) == (ln_b == nullptr), DSA_ERR_INVALID_ARG,
              "dsa_indexer_store: ln_w and ln_b must both be given or both be NULL");
  DSA_REQUIRE(eps >= 0.f, DSA_ERR_INVALID_ARG, "dsa_indexer_store: eps < 0");
  if (B == 0) return DSA_OK;
  DSA_REQUIRE(k_new && gate_new && pos && tok_off && k && gate && valid, DSA_ERR_INVALID_ARG,
              "dsa_indexer_store: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_indexer_store", k_new, gate_new, pos, tok_off, ln_w, ln_b, k, gate,
                      valid);
  const int lpp = D / 8, per_wg = 256 / lpp;
  const dim3 grid((B + per_wg - 1) / per_wg);
  if (dsa::dry_run()) return DSA_OK;
#define DSA_LAUNCH_STORE(LPP)                                                                  \
  indexer_store_kernel<LPP><<<grid, 256, 0, stream>>>(k_new, gate_new, pos, tok_off, ln_w, ln_b, \
                                                      eps, B, k, gate, valid)
  switch (lpp) {
    case 4: DSA_LAUNCH_STORE(4); break;
    case 8: DSA_LAUNCH_STORE(8); break;
    case 16: DSA_LAUNCH_STORE(16); break;
    default: DSA_LAUNCH_STORE(32); break;
  }
#undef DSA_LAUNCH_STORE
  return dsa::check_launch("dsa_indexer_store");
}
