// a4: pool top-k with lowest-id tie-breaking, emitted in ascending pool id.
//
// One workgroup per score row (1024 threads, or 256 for rows of at most 1024
// pools); thread t holds ids t + NT*e (e < E), so every load instruction is
// fully coalesced and the order (e, t) is ascending id order.  Scores become
// order-preserving integer keys (a finite float maps to a nonzero unsigned
// key that sorts like the float; -0 like +0; non-candidates are key 0 and
// never counted), so no floating-point comparison decides the selection.
//  1. Candidate count and largest key (wave ballots / DPP max, one barrier).
//  2. Octave of every key below the largest (difference of the top 9 key bits
//     = sign and exponent, capped at 15), counted in packed 8-bit register
//     fields and summed over the workgroup in a fixed order -- no atomics,
//     because nearly all scores of a row share their top key bits.
//  3. Inside the octave holding the k_eff-th best key, byte-wise radix passes
//     over per-wave LDS histograms pin the threshold key T (stopping early
//     once the threshold bin is taken whole).
//  4. Keys above T are kept and, among keys equal to T, the lowest ids (a
//     rank pass only when the budget splits one key value); kept ids are
//     compacted in id order with wave ballots and per-(e, wave) offsets that
//     one wave scans.
// The fused variant (dsa_topk_expand) also writes the expanded token ids of
// each kept pool (a5): the pools' start rows are loaded beside the scores, so
// the expansion adds no dependent load and no launch.
#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

// Rows of more than kShortRow pools take 1024-thread workgroups; shorter rows
// (prefill: thousands of rows of at most a thousand pools) take 256 threads,
// so that several rows share a compute unit and fewer waves meet at each
// barrier.
constexpr int kShortRow = 1024;
constexpr int kStage = 2048;  // largest select_k whose output is staged in LDS

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
// number of set bits of m below this lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Expansion arguments of the fused variant (a5): token row of each kept pool.
struct ExpandArgs {
  const int32_t* pool_start;
  const int32_t* pool_off;
  const int32_t* q_req;
  int kpool, out_width;
  int32_t* tok;
};

// Exclusive prefix, in (e, wave) order, of the per-(e, wave) counts in cnt
// (E * NW entries), written to off; run by wave 0 alone.
template <int E, int NW>
__device__ __forceinline__ void wave0_offsets(const int* __restrict__ cnt, int* __restrict__ off,
                                              int lane) {
  constexpr int kN = E * NW;
  constexpr int kPer = (kN + 63) / 64;
  int c[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ix = lane * kPer + i;
    c[i] = ix < kN ? cnt[ix] : 0;
    sum += c[i];
  }
  int base = wave_incl_scan(sum) - sum;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ix = lane * kPer + i;
    if (ix < kN) off[ix] = base;
    base += c[i];
  }
}

template <int NT, int E, bool EXPAND>  // NT threads per row, E ids per thread
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores,
                                                        const uint8_t* __restrict__ cand,
                                                        const int32_t* __restrict__ row_len,
                                                        int pstride, int select_k,
                                                        int32_t* __restrict__ sel, ExpandArgs ex) {
  constexpr int kThreads = NT, kWaves = NT / 64;
  static_assert(NT >= 256, "the radix bins are summed by one thread each");
  __shared__ int hist[kWaves][256];
  __shared__ int s_tot[256];
  __shared__ uint32_t s_max[kWaves];
  __shared__ int s_cnt[kWaves];
  __shared__ int s_oct[kWaves][16];
  __shared__ int s_ecnt[E * kWaves];  // per (e, wave) counts
  __shared__ int s_eoff[E * kWaves];  // their exclusive prefix in (e, wave) order
  __shared__ int s_bin, s_above, s_binc;
  // kept ids and their start rows in output order (when select_k <= kStage),
  // written out coalesced
  __shared__ int s_kid[kStage], s_kps[EXPAND ? kStage : 1];
  const int q = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const float* srow = scores + (int64_t)q * pstride;
  const uint8_t* crow = cand + (int64_t)q * pstride;
  int32_t* out = sel + (int64_t)q * select_k;

  // loads (ids clamped into the row), then masked; the row's length loads
  // beside them (without row_len it reads a score word and does not use it)
  float sv[E];
  uint8_t cv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // (unsigned, so the address is a 32-bit offset from the row's base)
    const unsigned id = min((unsigned)(t + kThreads * e), (unsigned)(pstride - 1));
    sv[e] = srow[id];
    cv[e] = crow[id];
  }
  const int len_word = *(row_len ? row_len + q : (const int32_t*)srow);
  // fused expansion: start rows of this request's pool slots, loaded without a
  // branch (ids clamped to the request's slots; a request with no slot reads
  // q_req instead, and none of its pools can be selected)
  int32_t ps[EXPAND ? E : 1];
  int32_t* trow = nullptr;
  if (EXPAND) {
    const int r = ex.q_req[q];
    const int pb = ex.pool_off[r], cap = ex.pool_off[r + 1] - pb;
    trow = ex.tok + (int64_t)q * ex.out_width;
    const int32_t* src = cap > 0 ? ex.pool_start + pb : ex.q_req;
    const int last = max(cap - 1, 0);
#pragma unroll
    for (int e = 0; e < E; ++e) ps[e] = src[min(t + kThreads * e, last)];
  }
  const int lenq = row_len ? min(max(len_word, 0), pstride) : pstride;  // entries that count
  uint32_t key[E];
  uint32_t kmx = 0u;
  int nc = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // the empty asm hands the loaded values over as opaque registers, so the
    // compiler cannot turn the masking below into a branch around a load
    // (which would end in a wait for every outstanding load)
    uint32_t u = __float_as_uint(sv[e]), cb = cv[e];
    asm volatile("" : "+v"(u), "+v"(cb));
    const bool c = (t + kThreads * e < lenq) & (cb != 0u);
    key[e] = c ? float_order_key(__uint_as_float(u)) : 0u;
    kmx = max(kmx, key[e]);
    nc += __popcll(ballot(key[e] != 0u));  // (no candidate's key is 0)
  }
  kmx = wave_max_u32(kmx);
  if (lane == 0) {
    s_max[wv] = kmx;
    s_cnt[wv] = nc;
  }
  __syncthreads();
  int ncand = 0;
  uint32_t kmax = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    ncand += s_cnt[w];
    kmax = max(kmax, s_max[w]);
  }
  const int k_eff = min(select_k, ncand);
  if (k_eff == 0) {
    for (int i = t; i < select_k; i += kThreads) out[i] = -1;
    if (EXPAND)
      for (int i = t; i < ex.out_width; i += kThreads) trow[i] = -1;
    return;
  }
  const uint32_t top9 = kmax >> 23;

  // 2. octave counts: 16 four-bit counters per 64-bit word, one word per 8
  // keys (so no counter exceeds 8), widened to 16-bit pairs
  uint32_t oct[E];
  uint32_t p[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int e0 = 0; e0 < E; e0 += 8) {
    uint64_t c4 = 0ull;
#pragma unroll
    for (int e = e0; e < e0 + 8 && e < E; ++e) {
      const uint32_t d = min(top9 - (key[e] >> 23), 15u);
      oct[e] = key[e] ? d : 16u;
      c4 += key[e] ? (1ull << (4u * d)) : 0ull;
    }
    const uint32_t lo = (uint32_t)c4, hi = (uint32_t)(c4 >> 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] += ((lo >> (8 * j)) & 0xFu) | (((lo >> (8 * j + 4)) & 0xFu) << 16);
      p[4 + j] += ((hi >> (8 * j)) & 0xFu) | (((hi >> (8 * j + 4)) & 0xFu) << 16);
    }
  }
  {
    // reduce-scatter the 8 pairs (bins 2j, 2j+1) over the wave (fields stay below 2^16)
    int v4[4], v2[2], v1;
    {
      const bool hi = (lane >> 5) & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v4[i] = (int)(hi ? p[4 + i] : p[i]) + xor32_i((int)(hi ? p[i] : p[4 + i]));
    }
    {
      const bool hi = (lane >> 4) & 1;
#pragma unroll
      for (int i = 0; i < 2; ++i) v2[i] = (hi ? v4[2 + i] : v4[i]) + xor16_i(hi ? v4[i] : v4[2 + i]);
    }
    {
      const bool hi = (lane >> 3) & 1;
      v1 = (hi ? v2[1] : v2[0]) + dpp_i<kDppMirror>(hi ? v2[0] : v2[1]);
    }
    v1 += dpp_i<kDppHalfMirror>(v1);
    v1 += dpp_i<kDppXor2>(v1);
    v1 += dpp_i<kDppXor1>(v1);
    if ((lane & 7) == 0) {
      const int j = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
      s_oct[wv][2 * j] = v1 & 0xffff;
      s_oct[wv][2 * j + 1] = (int)((uint32_t)v1 >> 16);
    }
  }
  __syncthreads();
  if (t < 64) {
    int tot = 0;
    if (t < 16)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += s_oct[w][t];
    const int x = wave_incl_scan(tot);  // octaves 0..15, nearest the max first
    const int before = x - tot;
    if (t < 16 && before < k_eff && k_eff <= x) {
      s_bin = t;
      s_above = before;
      s_binc = tot;
    }
  }
  __syncthreads();
  const uint32_t boct = (uint32_t)s_bin;
  int krem = k_eff - s_above;
  int binc = s_binc;
  // the threshold octave; octave 15 also holds everything further down
  uint32_t prefix = boct < 15u ? (top9 - boct) << 23 : 0u;
  uint32_t mask = boct < 15u ? 0xFF800000u : 0u;
  bool act[E];
#pragma unroll
  for (int e = 0; e < E; ++e) act[e] = boct < 15u ? oct[e] == boct : (oct[e] >= 15u && oct[e] < 16u);

  // 3. byte-wise radix passes inside the threshold octave
  if (binc != krem) {
    for (int hi = boct < 15u ? 22 : 31; hi >= 0; hi -= 8) {
      const int lo = hi >= 7 ? hi - 7 : 0;
      const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
      for (int i = lane; i < 256; i += 64) hist[wv][i] = 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (act[e] && (key[e] & mask) == prefix) atomicAdd(&hist[wv][(key[e] >> lo) & dmask], 1);
      __syncthreads();
      if (t < 256) {
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += hist[w][t];
        s_tot[t] = tot;
      }
      __syncthreads();
      if (t < 64) {
        // lane t holds bins 255-4t .. 252-4t (descending): an inclusive prefix
        // over lanes counts the keys in higher bins
        int h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = s_tot[255 - 4 * t - j];
        const int sl = h[0] + h[1] + h[2] + h[3];
        int above = wave_incl_scan(sl) - sl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above < krem && krem <= above + h[j]) {
            s_bin = 255 - 4 * t - j;
            s_above = above;
            s_binc = h[j];
          }
          above += h[j];
        }
      }
      __syncthreads();
      const int b = s_bin;
      binc = s_binc;
      krem -= s_above;
      prefix |= (uint32_t)b << lo;
      mask |= dmask << lo;
      if (binc == krem) break;  // the whole threshold bin is taken
    }
  }

  if (EXPAND) {
    // take delivery of the start rows here, before the stores, so that no
    // wait inside the store phase covers the stores themselves
#pragma unroll
    for (int e = 0; e < E; ++e) asm volatile("" ::"v"(ps[e]));
  }
  // 4. keys above the threshold bin are kept, and from the bin either all of
  // it or, when its keys are one value split by the budget, the lowest ids
  bool keep[E];
  if (binc == krem) {
#pragma unroll
    for (int e = 0; e < E; ++e) keep[e] = oct[e] < boct || (act[e] && (key[e] & mask) >= prefix);
  } else {
    bool gt[E], eq[E];
    uint64_t beq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t km = key[e] & mask;
      gt[e] = oct[e] < boct || (act[e] && km > prefix);
      eq[e] = act[e] && km == prefix;
      beq[e] = ballot(eq[e]);
      if (lane == 0) s_ecnt[e * kWaves + wv] = __popcll(beq[e]);
    }
    __syncthreads();
    if (wv == 0) wave0_offsets<E, kWaves>(s_ecnt, s_eoff, lane);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      keep[e] = gt[e] || (eq[e] && s_eoff[e * kWaves + wv] + lanes_below(beq[e]) < krem);
    __syncthreads();  // s_ecnt / s_eoff are reused below
  }
  // compaction of the kept ids in id order: (e, wave, lane) is ascending id
  uint64_t bk[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bk[e] = ballot(keep[e]);
    if (lane == 0) s_ecnt[e * kWaves + wv] = __popcll(bk[e]);
  }
  __syncthreads();
  if (wv == 0) wave0_offsets<E, kWaves>(s_ecnt, s_eoff, lane);
  __syncthreads();
  if (select_k <= kStage) {
    // positions into LDS, then every output row written in order by all threads
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int pos = s_eoff[e * kWaves + wv] + lanes_below(bk[e]);
      if (keep[e] && pos < k_eff) {
        s_kid[pos] = t + kThreads * e;
        if (EXPAND) s_kps[pos] = ps[e];
      }
    }
    __syncthreads();
    for (int i = t; i < select_k; i += kThreads) out[i] = i < k_eff ? s_kid[i] : -1;
    if (EXPAND) {
      const int kp = ex.kpool;
      for (int i = t; i < ex.out_width; i += kThreads) {
        const int j = i / kp;
        trow[i] = j < k_eff ? s_kps[j] + (i - j * kp) : -1;
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int pos = s_eoff[e * kWaves + wv] + lanes_below(bk[e]);
    if (keep[e] && pos < k_eff) {
      out[pos] = t + kThreads * e;
      if (EXPAND) {
#pragma unroll
        for (int s = 0; s < DSA_MAX_KPOOL; ++s)
          if (s < ex.kpool) trow[pos * ex.kpool + s] = ps[e] + s;
      }
    }
  }
  for (int i = k_eff + t; i < select_k; i += kThreads) out[i] = -1;
  if (EXPAND)
    for (int i = k_eff * ex.kpool + t; i < ex.out_width; i += kThreads) trow[i] = -1;
}

template <bool EXPAND>
dsa_status launch_topk(const float* scores, const uint8_t* cand, const int32_t* row_len, int Q,
                       int pstride, int select_k,
                       int32_t* sel, const ExpandArgs& ex, hipStream_t stream) {
  const int nt = pstride <= kShortRow ? 256 : 1024;
  const int need = (pstride + nt - 1) / nt;
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] topk_pools Q=%d pstride=%d select_k=%d threads=%d E=%d expand=%d\n", Q,
            pstride, select_k, nt, need, (int)EXPAND);
#define DSA_LAUNCH_TK(NT, E)                                                                     \
  topk_kernel<NT, E, EXPAND><<<Q, NT, 0, stream>>>(scores, cand, row_len, pstride, select_k, sel, \
                                                   ex)
  if (nt == 256) {
    if (need <= 1) DSA_LAUNCH_TK(256, 1);
    else if (need <= 2) DSA_LAUNCH_TK(256, 2);
    else DSA_LAUNCH_TK(256, 4);
  } else {
    if (need <= 1) DSA_LAUNCH_TK(1024, 1);
    else if (need <= 2) DSA_LAUNCH_TK(1024, 2);
    else if (need <= 4) DSA_LAUNCH_TK(1024, 4);
    else if (need <= 8) DSA_LAUNCH_TK(1024, 8);
    else DSA_LAUNCH_TK(1024, 16);
  }
#undef DSA_LAUNCH_TK
  return dsa::check_launch(EXPAND ? "dsa_topk_expand" : "dsa_topk_pools");
}

}  // namespace

DSA_EXPORT size_t dsa_topk_pools_workspace_size(int Q, int pstride, int select_k) {
  (void)Q;
  (void)pstride;
  (void)select_k;
  return 0;
}

DSA_EXPORT dsa_status dsa_topk_pools(const float* scores, const uint8_t* cand,
                                     const int32_t* row_len, int Q, int pstride, int select_k,
                                     int32_t* sel, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  DSA_REQUIRE(select_k >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_pools: select_k=%d < 1", select_k);
  DSA_REQUIRE(pstride >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_pools: pstride=%d < 1", pstride);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "dsa_topk_pools: Q=%d < 0", Q);
  DSA_REQUIRE(pstride <= DSA_MAX_TOPK_ROW, DSA_ERR_UNSUPPORTED,
              "dsa_topk_pools: pstride=%d above %d", pstride, DSA_MAX_TOPK_ROW);
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(scores && cand && sel, DSA_ERR_INVALID_ARG, "dsa_topk_pools: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_topk_pools", scores, cand, row_len, sel, ws);
  return launch_topk<false>(scores, cand, row_len, Q, pstride, select_k, sel, ExpandArgs{},
                            stream);
}

DSA_EXPORT dsa_status dsa_topk_expand(const float* scores, const uint8_t* cand,
                                      const int32_t* row_len, int Q, int pstride, int select_k,
                                      const int32_t* pool_start,
                                      const int32_t* pool_off, const int32_t* q_req, int kpool,
                                      int out_width, int flags, int32_t* sel, int32_t* tok,
                                      hipStream_t stream) {
  DSA_REQUIRE(select_k >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_expand: select_k=%d < 1", select_k);
  DSA_REQUIRE(pstride >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_expand: pstride=%d < 1", pstride);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "dsa_topk_expand: Q=%d < 0", Q);
  DSA_REQUIRE(pstride <= DSA_MAX_TOPK_ROW, DSA_ERR_UNSUPPORTED,
              "dsa_topk_expand: pstride=%d above %d", pstride, DSA_MAX_TOPK_ROW);
  DSA_REQUIRE((flags & ~1) == 0, DSA_ERR_INVALID_ARG, "dsa_topk_expand: unknown flags 0x%x",
              flags);
  DSA_REQUIRE((flags & 1) == 0, DSA_ERR_UNSUPPORTED,
              "dsa_topk_expand: flag bit 0 is reserved (dsa_select_tail writes the tail)");
  DSA_REQUIRE(kpool >= 1 && kpool <= DSA_MAX_KPOOL, DSA_ERR_INVALID_ARG,
              "dsa_topk_expand: kpool=%d outside [1,%d]", kpool, DSA_MAX_KPOOL);
  DSA_REQUIRE((long long)out_width >= (long long)select_k * kpool, DSA_ERR_INVALID_ARG,
              "dsa_topk_expand: out_width=%d < select_k*kpool=%lld", out_width,
              (long long)select_k * kpool);
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(scores && cand && sel && pool_start && pool_off && q_req && tok,
              DSA_ERR_INVALID_ARG, "dsa_topk_expand: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_topk_expand", scores, cand, row_len, pool_start, pool_off, q_req, sel,
                      tok);
  return launch_topk<true>(scores, cand, row_len, Q, pstride, select_k, sel,
                           ExpandArgs{pool_start, pool_off, q_req, kpool, out_width, tok}, stream);
}
