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
              "dsa_expand_selection: always_select_tail is not built");
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
  dim3 grid((out_width + 255) / 256, Q);
  expand_kernel<<<grid, 256, 0, stream>>>(sel, pool_start, pool_off, q_req, select_k, kpool,
                                          out_width, tok);
  return dsa::check_launch("dsa_expand_selection");
}
