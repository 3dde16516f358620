// a5: selection expansion  tok[q, j*kpool + s] = pool_start[sel[q,j]] + s.
//
// Atlas glm5next_dsa page, "Traps carried from Slice 8": the -1 sentinel
// destination must be fully written (an unwritten tail of an uninitialised
// buffer once became "token indices").  One thread per output element, so
// every element of every row is stored exactly once.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

__global__ __launch_bounds__(256) void expand_kernel(const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ pool_start,
                                                     const int32_t* __restrict__ pool_off,
                                                     const int32_t* __restrict__ q_req,
                                                     int select_k, int kpool, int out_width,
                                                     int32_t* __restrict__ tok) {
  const int q = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= out_width) return;
  const int j = i / kpool, s = i - j * kpool;
  int v = -1;
  if (j < select_k) {
    const int p = sel[(int64_t)q * select_k + j];
    if (p >= 0) v = pool_start[(int64_t)pool_off[q_req[q]] + p] + s;
  }
  tok[(int64_t)q * out_width + i] = v;
}

}  // namespace

DSA_EXPORT dsa_status dsa_expand_selection(const int32_t* sel, const int32_t* pool_start,
                                           const int32_t* pool_off, const int32_t* q_req, int Q,
                                           int select_k, int kpool, int out_width, int flags,
                                           int32_t* tok, hipStream_t stream) {
  DSA_REQUIRE((flags & ~1) == 0, DSA_ERR_INVALID_ARG, "dsa_expand_selection: unknown flags 0x%x",
              flags);
  DSA_REQUIRE((flags & 1) == 0, DSA_ERR_UNSUPPORTED,
              "dsa_expand_selection: flag bit 0 is reserved (dsa_select_tail writes the tail)");
  DSA_REQUIRE(kpool >= 1 && kpool <= DSA_MAX_KPOOL, DSA_ERR_INVALID_ARG,
              "dsa_expand_selection: kpool=%d outside [1,%d]", kpool, DSA_MAX_KPOOL);
  DSA_REQUIRE(select_k >= 1, DSA_ERR_INVALID_ARG, "dsa_expand_selection: select_k=%d < 1",
              select_k);
  DSA_REQUIRE((long long)out_width >= (long long)select_k * kpool, DSA_ERR_INVALID_ARG,
              "dsa_expand_selection: out_width=%d < select_k*kpool=%lld", out_width,
              (long long)select_k * kpool);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "dsa_expand_selection: Q=%d < 0", Q);
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(sel && pool_start && pool_off && q_req && tok, DSA_ERR_INVALID_ARG,
              "dsa_expand_selection: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_expand_selection", sel, pool_start, pool_off, q_req, tok);
  DSA_REQUIRE(Q <= 65535, DSA_ERR_UNSUPPORTED, "dsa_expand_selection: Q=%d above 65535", Q);
  dim3 grid((out_width + 255) / 256, Q);
  if (dsa::dry_run()) return DSA_OK;
  expand_kernel<<<grid, 256, 0, stream>>>(sel, pool_start, pool_off, q_req, select_k, kpool,
                                          out_width, tok);
  return dsa::check_launch("dsa_expand_selection");
}

// always_select_tail (Atlas glm5next_dsa page, Glm5NextDsaConfig::out_width:
// the tail adds kpool-1 slots to the emitted row).  For a query at position t
// of request r with first valid row f, the pools that count for it end at or
// before t; the rows after them up to t -- fewer than kpool -- are its tail,
// and its valid rows go, in order, to the kpool-1 slots after the
// select_k*kpool pool slots.  f is pool 0's start when the request has a pool;
// without one, every valid row of the request lies within the last kpool-1
// rows, so the window t-kpool+2 .. t holds the whole tail.  One thread per query.
namespace {

__global__ __launch_bounds__(64) void tail_kernel(const uint8_t* __restrict__ valid,
                                                  const int32_t* __restrict__ tok_off,
                                                  const int32_t* __restrict__ pool_start,
                                                  const int32_t* __restrict__ pool_off,
                                                  const int32_t* __restrict__ n_pools,
                                                  const int32_t* __restrict__ q_req,
                                                  const int32_t* __restrict__ q_pos, int Q,
                                                  int kpool, int select_k, int out_width,
                                                  int32_t* __restrict__ tok) {
  const int q = blockIdx.x * 64 + threadIdx.x;
  if (q >= Q) return;
  const int r = q_req[q], t = q_pos[q];
  const int64_t row0 = tok_off[r];
  const int np = n_pools[r];
  int lo;
  if (np > 0) {
    const int f = pool_start[pool_off[r]];
    lo = t >= f ? f + ((t + 1 - f) / kpool) * kpool : t + 1;
  } else {
    lo = max(0, t - kpool + 2);
  }
  int32_t* out = tok + (int64_t)q * out_width + (int64_t)select_k * kpool;
  int n = 0;
  for (int x = lo; x <= t; ++x)
    if (valid[row0 + x]) out[n++] = x;
  for (; n < kpool - 1; ++n) out[n] = -1;
}

}  // namespace

DSA_EXPORT dsa_status dsa_select_tail(const uint8_t* valid, const int32_t* tok_off,
                                      const int32_t* pool_start, const int32_t* pool_off,
                                      const int32_t* n_pools, const int32_t* q_req,
                                      const int32_t* q_pos, int Q, int kpool, int select_k,
                                      int out_width, int32_t* tok, hipStream_t stream) {
  DSA_REQUIRE(kpool >= 1 && kpool <= DSA_MAX_KPOOL, DSA_ERR_INVALID_ARG,
              "dsa_select_tail: kpool=%d outside [1,%d]", kpool, DSA_MAX_KPOOL);
  DSA_REQUIRE(select_k >= 1, DSA_ERR_INVALID_ARG, "dsa_select_tail: select_k=%d < 1", select_k);
  DSA_REQUIRE((long long)out_width >= (long long)select_k * kpool + kpool - 1,
              DSA_ERR_INVALID_ARG,
              "dsa_select_tail: out_width=%d < select_k*kpool + kpool-1 = %lld", out_width,
              (long long)select_k * kpool + kpool - 1);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "dsa_select_tail: Q=%d < 0", Q);
  if (Q == 0 || kpool == 1) return DSA_OK;  // kpool 1: no tail slots
  DSA_REQUIRE(valid && tok_off && pool_start && pool_off && n_pools && q_req && q_pos && tok,
              DSA_ERR_INVALID_ARG, "dsa_select_tail: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_select_tail", valid, tok_off, pool_start, pool_off, n_pools, q_req,
                      q_pos, tok);
  if (dsa::dry_run()) return DSA_OK;
  tail_kernel<<<(Q + 63) / 64, 64, 0, stream>>>(valid, tok_off, pool_start, pool_off, n_pools,
                                                q_req, q_pos, Q, kpool, select_k, out_width, tok);
  return dsa::check_launch("dsa_select_tail");
}
