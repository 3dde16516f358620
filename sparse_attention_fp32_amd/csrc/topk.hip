// a4: pool top-k with lowest-id tie-breaking, emitted in ascending pool id.
//
// One workgroup per score row (1024 threads, or 256 for rows of at most 1024
// pools).  Thread t holds ids t + NT*e of a pass step of NT*E ids, so every
// load instruction is fully coalesced and the order (step, e, t) is ascending
// id order.  A row that does not fit one step (more than 16384 pools) is
// selected in two launches when there is room for the candidates (each block
// of the row keeps its own top-k, then one workgroup selects among them; see
// TwoStage), else read again from memory (L2) on every pass instead of staying
// in registers; there is no cap on the row length.  A row that fits one step
// but keeps at most an eighth of each 2048-pool block takes the two launches
// as well (stage_blk).
//
// Scores become order-preserving integer keys (a finite float maps to a
// nonzero unsigned key that sorts like the float; -0 like +0; non-candidates
// are key 0 and never counted), so no floating-point comparison decides the
// selection.  The threshold -- the key of the k_eff-th best candidate -- is
// found by a most-significant-digit radix select with three digits of 11, 11
// and 10 bits:
//  * one pass counts the candidates whose key starts with the digits found so
//    far, by their next digit, in a 2048-bin LDS histogram (a wave whose
//    counted keys all share one digit adds them with one atomic, so ties and
//    clusters do not serialise the LDS);
//  * a scan over the bins, highest first, finds the digit whose bin holds the
//    k_eff-th best candidate; when that bin is taken whole the select stops
//    early (the usual case after the first or second digit on real scores).
// Keys above the threshold are kept; among keys equal to a threshold that the
// budget splits, the lowest ids (a rank pass over equal keys in id order).
// Kept ids are compacted in id order with wave ballots and per-(e, wave)
// offsets that one wave scans, staged in LDS and written out coalesced.
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
constexpr int kBins = 2048;  // radix digits of 11 bits (the last digit has 10)

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

// Long rows in two stages.  Stage 1 (MODE 1): workgroup (row q, block b)
// selects the block's own top select_k among ids [b*blk, (b+1)*blk) -- the
// row's top select_k is among the union of the blocks' (every id that beats
// it in the row's order beats it in its block's too) -- and writes their row
// ids, ascending, -1-padded, to ids[q*stride + b*select_k ..].  Stage 2
// (MODE 2): one workgroup per row selects among those ncand = nblk*select_k
// candidates, keyed by the row's own scores, and emits their ids; positions
// ascend with the ids, so ties still go to the lower id.
struct TwoStage {
  int32_t* ids;  // [Q, stride] candidate ids (stage 1 writes, stage 2 reads)
  int stride;
  int blk;       // block length (stage 1)
  int ncand;     // candidates per row (stage 2)
};

// Exclusive prefix, in (e, wave) order, of the per-(e, wave) counts in cnt
// (E * NW entries), written to off, plus `base`; returns the total (in every
// lane).  Run by wave 0 alone.
template <int E, int NW>
__device__ __forceinline__ int wave0_offsets(const int* __restrict__ cnt, int* __restrict__ off,
                                             int lane, int base) {
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
  const int incl = wave_incl_scan(sum);
  int run = base + incl - sum;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ix = lane * kPer + i;
    if (ix < kN) off[ix] = run;
    run += c[i];
  }
  return __builtin_amdgcn_readlane(incl, 63);
}

// Adds 1 to h[bin] for every lane with `pred`; when every such lane of the
// wave has the same bin, one lane adds their count.
__device__ __forceinline__ void hist_add(int* h, bool pred, uint32_t bin) {
  const uint64_t act = ballot(pred);
  if (act == 0ull) return;
  const int first = __builtin_ctzll(act);
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
  if (ballot(pred && bin == b0) == act) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&h[b0], (int)__popcll(act));
  } else if (pred) {
    atomicAdd(&h[bin], 1);
  }
}

// NT threads per row, E ids per thread per step; MODE 0: the row itself,
// 1: a block of it (stage 1), 2: the candidates of stage 1 (stage 2)
template <int NT, int E, bool STREAM, bool EXPAND, int MODE = 0>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores,
                                                  const uint8_t* __restrict__ cand,
                                                  const int32_t* __restrict__ row_len,
                                                  int pstride, int select_k,
                                                  int32_t* __restrict__ sel, ExpandArgs ex,
                                                  TwoStage ts) {
  static_assert(MODE == 0 || (!STREAM && (MODE == 2 || !EXPAND)), "two-stage modes");
  constexpr int kWaves = NT / 64;
  constexpr int kStep = NT * E;
  constexpr int kBpt = kBins / NT;  // histogram bins per thread in the scan
  // kept ids and their start rows in output order (when k_eff <= kStage), written
  // out coalesced; a row of a 256-thread workgroup holds at most 1024 candidates
  constexpr int kStage = NT == 256 ? kShortRow : 2048;
  static_assert(kBins % NT == 0, "bins per thread");
  __shared__ int hist[2][kBins];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_res[3];            // digit, keys above its bin, keys in its bin
  __shared__ int s_ecnt[E * kWaves];  // per (e, wave) counts
  __shared__ int s_eoff[E * kWaves];  // their exclusive prefix in (e, wave) order
  __shared__ int s_run[2];            // kept / equal keys of earlier steps (long rows)
  __shared__ int s_kid[kStage], s_kps[EXPAND ? kStage : 1];
  const int q = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // stage 1: this workgroup's block is ids [id0, id0 + plen) of the row
  const int id0 = MODE == 1 ? (int)blockIdx.y * ts.blk : 0;
  const int plen = MODE == 1 ? min(ts.blk, pstride - id0) : (MODE == 2 ? ts.ncand : pstride);
  const float* srow = scores + (int64_t)q * pstride + id0;
  const uint8_t* crow = cand + (int64_t)q * pstride + id0;
  const int32_t* cids = MODE == 2 ? ts.ids + (int64_t)q * ts.stride : nullptr;
  int32_t* out = MODE == 1 ? ts.ids + (int64_t)q * ts.stride + (int64_t)blockIdx.y * select_k
                           : sel + (int64_t)q * select_k;
  const int nstep = STREAM ? (pstride + kStep - 1) / kStep : 1;

  // fused expansion: the request's pool slots (a request with no slot reads
  // q_req instead, and none of its pools can be selected)
  const int32_t* psrc = nullptr;
  int pslast = 0;
  int32_t* trow = nullptr;
  if (EXPAND) {
    const int r = ex.q_req[q];
    const int pb = ex.pool_off[r], cap = ex.pool_off[r + 1] - pb;
    trow = ex.tok + (int64_t)q * ex.out_width;
    psrc = cap > 0 ? ex.pool_start + pb : ex.q_req;
    pslast = max(cap - 1, 0);
  }
  // the row's length loads beside the first scores (without row_len it reads a
  // score word and does not use it)
  const int len_word = *(row_len ? row_len + q : (const int32_t*)scores);

  // keys of pass step s (ids clamped into the row, then masked); with EXPAND
  // and `starts`, the start rows of those pools too
  uint32_t key[E];
  int32_t ps[EXPAND ? E : 1];
  int32_t cid[MODE == 2 ? E : 1];  // stage 2: the row id of each candidate slot (-1: none)
  int lenq = plen;
  auto load_step = [&](int s, bool starts) {
    float sv[E];
    uint8_t cv[E];
    if (MODE == 2) {
#pragma unroll
      for (int e = 0; e < E; ++e) cid[e] = cids[min(t + NT * e, plen - 1)];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      // (unsigned, so the address is a 32-bit offset from the row's base when
      // the row fits one step)
      const unsigned id = MODE == 2 ? (unsigned)max(cid[e], 0)
                                    : min((unsigned)(s * kStep + t + NT * e), (unsigned)(plen - 1));
      sv[e] = srow[id];
      cv[e] = crow[id];
      if (EXPAND && starts)
        ps[e] = psrc[min(MODE == 2 ? (int)id : (int)(s * kStep + t + NT * e), pslast)];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      // the empty asm hands the loaded values over as opaque registers, so the
      // compiler cannot turn the masking below into a branch around a load
      // (which would end in a wait for every outstanding load)
      uint32_t u = __float_as_uint(sv[e]), cb = cv[e];
      asm volatile("" : "+v"(u), "+v"(cb));
      const bool c = (s * kStep + t + NT * e < lenq) & (cb != 0u) & (MODE != 2 || cid[e] >= 0);
      key[e] = c ? float_order_key(__uint_as_float(u)) : 0u;
    }
  };
  if (!STREAM) load_step(0, EXPAND);
#pragma unroll
  for (int j = 0; j < 2 * kBins / NT; ++j) (&hist[0][0])[t + j * NT] = 0;
  // (STREAM: the first pass loads its steps after the length is known)
  if (MODE == 0) lenq = row_len ? min(max(len_word, 0), pstride) : pstride;
  if (MODE == 1) lenq = row_len ? min(max(len_word - id0, 0), plen) : plen;
  if (!STREAM) {
    // the first load_step ran before the length was known: mask again
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = (t + NT * e < lenq) ? key[e] : 0u;
  }
  __syncthreads();

  // -- radix select of the threshold: digits [31:21], [20:10], [9:0] ---------
  // (levels 0 and 2 count into hist[0], level 1 into hist[1])
  uint32_t prefix = 0u, mask = 0u;  // digits found so far
  int need = 0;                     // candidates still to take from the current bin
  int binc = 0;                     // candidates in the current bin
  int k_eff = 0;
  for (int level = 0; level < 3; ++level) {
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const uint32_t dmask = level == 2 ? 0x3FFu : 0x7FFu;
    int* h = hist[level & 1];
    for (int s = 0; s < nstep; ++s) {
      if (STREAM) load_step(s, false);
#pragma unroll
      for (int e = 0; e < E; ++e)
        hist_add(h, key[e] != 0u && (key[e] & mask) == prefix, (key[e] >> shift) & dmask);
    }
    __syncthreads();
    // bins from the highest: thread t holds bins kBins-1-t*kBpt downwards
    int c[kBpt];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kBpt; ++j) {
      c[j] = h[kBins - 1 - t * kBpt - j];
      sum += c[j];
    }
    const int incl = wave_incl_scan(sum);
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    // the waves' totals in one read: lane w holds wave w's, and their
    // inclusive scan gives the row's total and this wave's exclusive prefix
    const int wx = wave_incl_scan(lane < kWaves ? s_wsum[lane] : 0);
    const int total = __builtin_amdgcn_readlane(wx, kWaves - 1);
    int above = incl - sum + (wv > 0 ? __builtin_amdgcn_readlane(wx, wv > 0 ? wv - 1 : 0) : 0);
    if (level == 0) {
      k_eff = min(select_k, total);  // total: the row's candidates
      need = k_eff;
      if (k_eff == 0) break;
      // hist[0] is read no more until level 2: clear it (level 1's barriers
      // order this before level 2's counts)
#pragma unroll
      for (int j = 0; j < kBins / NT; ++j) hist[0][t + j * NT] = 0;
    }
#pragma unroll
    for (int j = 0; j < kBpt; ++j) {
      if (above < need && need <= above + c[j]) {
        s_res[0] = kBins - 1 - t * kBpt - j;
        s_res[1] = above;
        s_res[2] = c[j];
      }
      above += c[j];
    }
    __syncthreads();
    prefix |= (uint32_t)s_res[0] << shift;
    mask |= dmask << shift;
    need -= s_res[1];
    binc = s_res[2];
    if (binc == need) break;  // the whole bin is taken
  }

  if (k_eff == 0) {
    for (int i = t; i < select_k; i += NT) out[i] = -1;
    if (EXPAND)
      for (int i = t; i < ex.out_width; i += NT) trow[i] = -1;
    return;
  }
  // the threshold bin is taken whole, or (all three digits found) the budget
  // takes the `need` lowest ids of the keys equal to the threshold
  const bool whole = binc == need;

  // -- keep and compaction, in id order --------------------------------------
  if (wv == 0 && lane < 2) s_run[lane] = 0;
  const bool staged = k_eff <= kStage;
  for (int s = 0; s < nstep; ++s) {
    if (STREAM) load_step(s, EXPAND);
    if (EXPAND && !STREAM) {
      // take delivery of the start rows here, before the stores, so that no
      // wait inside the store phase covers the stores themselves
#pragma unroll
      for (int e = 0; e < E; ++e) asm volatile("" ::"v"(ps[e]));
    }
    bool keep[E];
    if (whole) {
#pragma unroll
      for (int e = 0; e < E; ++e) keep[e] = key[e] != 0u && (key[e] & mask) >= prefix;
    } else {
      bool gt[E], eq[E];
      uint64_t beq[E];
      int qc = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        gt[e] = key[e] != 0u && key[e] > prefix;  // mask is all ones here
        eq[e] = key[e] != 0u && key[e] == prefix;
        beq[e] = ballot(eq[e]);
        qc = lane == e ? (int)__popcll(beq[e]) : qc;
      }
      if (lane < E) s_ecnt[lane * kWaves + wv] = qc;
      __syncthreads();
      if (wv == 0) {
        const int n = wave0_offsets<E, kWaves>(s_ecnt, s_eoff, lane, s_run[1]);
        if (lane == 0) s_run[1] += n;  // (wave 0 alone reads and writes s_run)
      }
      __syncthreads();
      const int qo = lane < E ? s_eoff[lane * kWaves + wv] : 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        keep[e] = gt[e] || (eq[e] && __builtin_amdgcn_readlane(qo, e) + lanes_below(beq[e]) < need);
      __syncthreads();  // s_ecnt / s_eoff are reused below
    }
    // the wave's E counts go out in one store (lane e holds count e), and
    // their offsets come back in one read
    uint64_t bk[E];
    int kc = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bk[e] = ballot(keep[e]);
      kc = lane == e ? (int)__popcll(bk[e]) : kc;
    }
    if (lane < E) s_ecnt[lane * kWaves + wv] = kc;
    __syncthreads();
    if (wv == 0) {
      const int n = wave0_offsets<E, kWaves>(s_ecnt, s_eoff, lane, s_run[0]);
      if (lane == 0) s_run[0] += n;  // (read by wave 0 alone, before the next step's barrier)
    }
    __syncthreads();
    const int ko = lane < E ? s_eoff[lane * kWaves + wv] : 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int pos = __builtin_amdgcn_readlane(ko, e) + lanes_below(bk[e]);
      const int id = MODE == 2 ? cid[e] : id0 + s * kStep + t + NT * e;
      if (keep[e] && pos < k_eff) {
        if (staged) {
          s_kid[pos] = id;
          if (EXPAND) s_kps[pos] = ps[e];
        } else {
          out[pos] = id;
          if (EXPAND) {
#pragma unroll
            for (int j = 0; j < DSA_MAX_KPOOL; ++j)
              if (j < ex.kpool) trow[pos * ex.kpool + j] = ps[e] + j;
          }
        }
      }
    }
    if (STREAM) __syncthreads();  // s_ecnt / s_eoff / s_run are reused by the next step
  }
  if (staged) {
    __syncthreads();
    for (int i = t; i < select_k; i += NT) out[i] = i < k_eff ? s_kid[i] : -1;
    if (EXPAND) {
      const int kp = ex.kpool;
      for (int i = t; i < ex.out_width; i += NT) {
        const int j = kp == 4 ? i >> 2 : i / kp;
        trow[i] = j < k_eff ? s_kps[j] + (i - j * kp) : -1;
      }
    }
    return;
  }
  for (int i = k_eff + t; i < select_k; i += NT) out[i] = -1;
  if (EXPAND)
    for (int i = k_eff * ex.kpool + t; i < ex.out_width; i += NT) trow[i] = -1;
}

constexpr int kBlk = 16384;  // stage-1 block: 1024 threads x 16 ids in registers
constexpr int kBlkSmall = 2048;  // stage-1 block of rows that fit one pass: 2 ids per thread

// Stage-1 block length of the two-stage select, or 0 for one pass.  Rows past
// one register pass always take it; a row that fits one pass takes it in
// 2048-pool blocks when each block keeps at most an eighth of its pools (the
// second launch then costs less than the first pass saves: measured on
// 16384-pool rows keeping 256; a block keeping a quarter was slower).
int stage_blk(int pstride, int select_k) {
  if (pstride > kBlk) return kBlk;
  if (pstride >= 2 * kBlkSmall && 8LL * select_k <= kBlkSmall) return kBlkSmall;
  return 0;
}

// Candidates per row of the two-stage select, or 0 where the row takes one
// pass or the candidates would not fit stage 2's registers.
long long two_stage_cands(int pstride, int select_k) {
  const int blk = stage_blk(pstride, select_k);
  if (blk == 0) return 0;
  const long long nblk = (pstride + blk - 1) / blk;
  const long long n = nblk * select_k;
  return n <= kBlk ? n : 0;
}

template <bool EXPAND>
dsa_status launch_topk(const float* scores, const uint8_t* cand, const int32_t* row_len, int Q,
                       int pstride, int select_k, int32_t* sel, const ExpandArgs& ex,
                       int32_t* cbuf, int cstride, hipStream_t stream) {
  const char* who = EXPAND ? "dsa_topk_expand" : "dsa_topk_pools";
  const long long ncand = two_stage_cands(pstride, select_k);
  if (ncand > 0 && cbuf && ncand <= cstride) {
    // long row in two stages: the blocks' own top-k, then one select over them
    const int blk = stage_blk(pstride, select_k);
    const int nblk = (pstride + blk - 1) / blk;
    DSA_REQUIRE(nblk <= 65535, DSA_ERR_UNSUPPORTED, "%s: pstride=%d in %d blocks", who, pstride,
                nblk);
    if (dsa::trace_enabled())
      fprintf(stderr, "[dsa] topk two-stage Q=%d pstride=%d select_k=%d blocks=%d cands=%lld\n",
              Q, pstride, select_k, nblk, ncand);
    const TwoStage ts{cbuf, cstride, blk, (int)ncand};
    if (dsa::dry_run()) return DSA_OK;
    if (blk == kBlk)
      topk_kernel<1024, 16, false, false, 1><<<dim3(Q, nblk), 1024, 0, stream>>>(
          scores, cand, row_len, pstride, select_k, sel, ExpandArgs{}, ts);
    else
      topk_kernel<1024, kBlkSmall / 1024, false, false, 1><<<dim3(Q, nblk), 1024, 0, stream>>>(
          scores, cand, row_len, pstride, select_k, sel, ExpandArgs{}, ts);
    dsa_status st = dsa::check_launch(who);
    if (st != DSA_OK) return st;
    const int need = (int)((ncand + 1023) / 1024);
#define DSA_LAUNCH_TK2(E) \
  topk_kernel<1024, E, false, EXPAND, 2><<<Q, 1024, 0, stream>>>(scores, cand, row_len, pstride, \
                                                                 select_k, sel, ex, ts)
    if (need <= 1) DSA_LAUNCH_TK2(1);
    else if (need <= 2) DSA_LAUNCH_TK2(2);
    else if (need <= 4) DSA_LAUNCH_TK2(4);
    else if (need <= 8) DSA_LAUNCH_TK2(8);
    else DSA_LAUNCH_TK2(16);
#undef DSA_LAUNCH_TK2
    return dsa::check_launch(who);
  }
  const int nt = pstride <= kShortRow ? 256 : 1024;
  const int need = (pstride + nt - 1) / nt;
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] topk_pools Q=%d pstride=%d select_k=%d threads=%d E=%d expand=%d\n", Q,
            pstride, select_k, nt, need, (int)EXPAND);
  if (dsa::dry_run()) return DSA_OK;
#define DSA_LAUNCH_TK(NT, E, S)                                                               \
  topk_kernel<NT, E, S, EXPAND><<<Q, NT, 0, stream>>>(scores, cand, row_len, pstride, select_k, \
                                                      sel, ex, TwoStage{})
  if (nt == 256) {
    if (need <= 1) DSA_LAUNCH_TK(256, 1, false);
    else if (need <= 2) DSA_LAUNCH_TK(256, 2, false);
    else DSA_LAUNCH_TK(256, 4, false);
  } else {
    if (need <= 1) DSA_LAUNCH_TK(1024, 1, false);
    else if (need <= 2) DSA_LAUNCH_TK(1024, 2, false);
    else if (need <= 4) DSA_LAUNCH_TK(1024, 4, false);
    else if (need <= 8) DSA_LAUNCH_TK(1024, 8, false);
    else if (need <= 16) DSA_LAUNCH_TK(1024, 16, false);
    else DSA_LAUNCH_TK(1024, 16, true);
  }
#undef DSA_LAUNCH_TK
  return dsa::check_launch(who);
}

}  // namespace

DSA_EXPORT size_t dsa_topk_pools_workspace_size(int Q, int pstride, int select_k) {
  if (Q <= 0 || pstride < 1 || select_k < 1) return 0;
  return (size_t)Q * (size_t)two_stage_cands(pstride, select_k) * sizeof(int32_t);
}

DSA_EXPORT dsa_status dsa_topk_pools(const float* scores, const uint8_t* cand,
                                     const int32_t* row_len, int Q, int pstride, int select_k,
                                     int32_t* sel, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  DSA_REQUIRE(select_k >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_pools: select_k=%d < 1", select_k);
  DSA_REQUIRE(pstride >= 1, DSA_ERR_INVALID_ARG, "dsa_topk_pools: pstride=%d < 1", pstride);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "dsa_topk_pools: Q=%d < 0", Q);
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(scores && cand && sel, DSA_ERR_INVALID_ARG, "dsa_topk_pools: NULL tensor pointer");
  DSA_REQUIRE_ALIGNED("dsa_topk_pools", scores, cand, row_len, sel, ws);
  // the two-stage select of long rows when the workspace holds its candidates
  const long long nc = two_stage_cands(pstride, select_k);
  const bool two = nc > 0 && ws && ws_bytes >= (size_t)Q * (size_t)nc * sizeof(int32_t);
  return launch_topk<false>(scores, cand, row_len, Q, pstride, select_k, sel, ExpandArgs{},
                            two ? (int32_t*)ws : nullptr, (int)nc, stream);
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
  // (a long row's stage-1 candidates go to its tok row when they fit it; the
  // second stage reads them all before it writes the row)
  return launch_topk<true>(scores, cand, row_len, Q, pstride, select_k, sel,
                           ExpandArgs{pool_start, pool_off, q_req, kpool, out_width, tok}, tok,
                           out_width, stream);
}
