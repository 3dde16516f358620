// a6: NoPE sparse MLA decode over the selected token ids.
//
// Atlas glm5next_dsa page: "Traps carried from Slice 8" (NoPE -- the 512-wide
// latent row is both key and value) and the MASKED_ATTN_MAX_KEYS note (a
// per-row gather of the selected ids is exactly the dense set-membership mask;
// the serving kernel keeps an online softmax and no full score row).
//
// Work split (flash-decoding): workgroup (chunk, head block, query) takes up to
// 64 heads of one query over one chunk of its selected ids; 4 waves own 16
// heads each.  The chunk's ids are staged in LDS first; the chunk is then
// walked in 32-token sub-chunks whose gathered latent rows (1 KiB each, one
// coalesced wave load per row, every load unconditional: ids outside the
// selection are redirected to a selected row and masked) are prefetched into
// registers one sub-chunk ahead, staged in LDS and shared by the 4 waves.
// Per sub-chunk and wave, on v_mfma_f32_16x16x32_bf16:
//   S^T[32 tok x 16 heads] = C[32 x 512] . Q^T   (C from LDS, Q in registers)
//   online softmax per head (log2 domain) with a lazily moved reference max
//   O += P[16 x 32] . C[32 x 512]
// Computing S transposed lets the accumulator of QK^T serve as the A operand
// of PV with no data movement: K index 8g+j of lane group g maps to token 4g+j
// (j < 4) or 16+4g+j-4.  The PV B operand needs 8 tokens of one dimension per
// lane; a lane reads 16 bytes (8 consecutive dims) of each of its 8 token rows
// and regroups the halves into 8 B operands, so output tile e of dim group G
// holds dims G*128 + 8c + e at lane column c, and each lane stores 8
// consecutive dims at once.
// fp8 latent rows are expanded to bf16 exactly on the way into LDS; the row
// scale multiplies the logits and the probabilities instead of the data.
// With more than one chunk, per-chunk (max, sum, unnormalised O) partials go
// to the workspace and mla_combine_kernel merges them in chunk order.
#include <limits.h>

#include "dsa_device.hpp"
#include "dsa_host.hpp"

namespace {

using namespace dsa;

constexpr int L = DSA_KV_LORA;
constexpr int kSub = 32;                 // tokens per sub-chunk
constexpr int kRowBytes = L * 2 + 16;    // LDS row stride: bf16 row + 16-byte pad
constexpr int kTargetWG = 256;           // aim for one workgroup per CU
constexpr int kMinSubPerChunk = 4;       // >= 128 ids per chunk keeps partials small
constexpr int kMaxTch = 2048;            // ids per chunk staged in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Chunking {
  int nchunks;
  int tch;  // ids per chunk (multiple of kSub)
};

Chunking mla_chunking(int Q, int Hm, int out_width) {
  const int nsub = (out_width + kSub - 1) / kSub;
  const int hb = (Hm + 63) / 64;
  const long long base = (long long)Q * hb;
  long long want = (kTargetWG + base - 1) / base;
  const int max_chunks = nsub / kMinSubPerChunk > 1 ? nsub / kMinSubPerChunk : 1;
  if (want > max_chunks) want = max_chunks;
  const int min_chunks = (nsub * kSub + kMaxTch - 1) / kMaxTch;
  if (want < min_chunks) want = min_chunks;
  if (want < 1) want = 1;
  const int spc = (int)((nsub + want - 1) / want);
  return {(nsub + spc - 1) / spc, spc * kSub};
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *(const uint4*)p; }

__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) {
  return (x & 0xffffu) | (y << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) {
  return (x >> 16) | (y & 0xffff0000u);
}

template <bool FP8>
__global__ __launch_bounds__(256) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ ckv_v,
    const float* __restrict__ ckv_scale, const int32_t* __restrict__ kv_off,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ tok, int Hm, int out_width,
    int tch, float sm_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_c[kSub * kRowBytes];
  __shared__ int s_id[kMaxTch];      // selected id per chunk position, -1 if none
  __shared__ float s_mul[kSub];      // logit multiplier per token: sm_scale*log2e*row scale
  __shared__ float s_scl[kSub];      // row scale (1 for bf16)
  __shared__ int s_ok[kSub];
  __shared__ int s_safe;             // some selected id of this chunk, or -1

  const int chunk = blockIdx.x, nchunks = gridDim.x, hb = blockIdx.y, qx = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int head0 = hb * 64 + wave * 16;
  const int r = q_req[qx];
  const int64_t rowbase = kv_off[r];
  const int j0 = chunk * tch;
  const int j1 = min(out_width, j0 + tch);
  const int nsub = j1 > j0 ? (j1 - j0 + kSub - 1) / kSub : 0;
  const int32_t* trow = tok + (int64_t)qx * out_width;

  // Stage the chunk's ids (one round trip) while the Q operand loads.
  if (t == 0) s_safe = -1;
  const int hq = head0 + col;
  bf16x8_t qb[16];
  {
    const uint16_t* qrow = q + ((int64_t)qx * Hm + (hq < Hm ? hq : Hm - 1)) * L + grp * 8;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const uint4 v = ldg16(qrow + kk * 32);
      qb[kk] = as_bf16x8(hq < Hm ? v : make_uint4(0, 0, 0, 0));
    }
  }
  __syncthreads();
  for (int i = t; i < nsub * kSub; i += 256) {
    const int j = j0 + i;
    const int id = trow[j < j1 ? j : j1 - 1];
    const int v = j < j1 ? id : -1;
    s_id[i] = v;
    if (v >= 0) atomicMax(&s_safe, v);
  }
  __syncthreads();
  const int safe = s_safe;

  f32x4_t o[4][8];  // [dim group G][tile e]: O[head grp*4+i][G*128 + 8*col + e]
#pragma unroll
  for (int G = 0; G < 4; ++G)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[G][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Gather mapping: bf16 rows are 64 x 16 B (one wave per row, 8 rows per
  // thread); fp8 rows are 32 x 16 B (half a wave per row, 4 rows per thread).
  constexpr int NPRE = FP8 ? 4 : 8;
  constexpr int kColU = FP8 ? 32 : 64;
  const int prow0 = t / kColU, pcu = t % kColU;
  constexpr int kRowStep = 256 / kColU;
  uint4 pre0[NPRE];

  auto gather = [&](int s, uint4 (&dst)[NPRE]) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int id = s_id[s * kSub + prow0 + i * kRowStep];
      const int64_t g = rowbase + (id >= 0 ? id : safe);
      dst[i] = FP8 ? ldg16((const uint8_t*)ckv_v + g * L + pcu * 16)
                   : ldg16((const uint16_t*)ckv_v + g * L + pcu * 8);
    }
  };

  const int nwork = safe >= 0 ? nsub : 0;  // a chunk with no selected id has no work
  if (nwork > 0) gather(0, pre0);

  // One sub-chunk: stage the prefetched rows, start the next gather, compute.
  auto step = [&](int s, uint4 (&cur)[NPRE]) {
    __syncthreads();  // every wave is done with the previous sub-chunk
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int row = prow0 + i * kRowStep;
      if (FP8) {
        const uint4 v = cur[i];
        const uint32_t w8[4] = {v.x, v.y, v.z, v.w};
        uint32_t o16[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t b0 = fp8e4m3_to_bf16(w8[k] & 0xffu);
          const uint32_t b1 = fp8e4m3_to_bf16((w8[k] >> 8) & 0xffu);
          const uint32_t b2 = fp8e4m3_to_bf16((w8[k] >> 16) & 0xffu);
          const uint32_t b3 = fp8e4m3_to_bf16(w8[k] >> 24);
          o16[2 * k] = b0 | (b1 << 16);
          o16[2 * k + 1] = b2 | (b3 << 16);
        }
        uint4* dst = (uint4*)(lds_c + row * kRowBytes + pcu * 32);
        dst[0] = make_uint4(o16[0], o16[1], o16[2], o16[3]);
        dst[1] = make_uint4(o16[4], o16[5], o16[6], o16[7]);
      } else {
        *(uint4*)(lds_c + row * kRowBytes + pcu * 16) = cur[i];
      }
    }
    if (t < kSub) {
      const int id = s_id[s * kSub + t];
      const float scl = FP8 ? ckv_scale[rowbase + (id >= 0 ? id : safe)] : 1.f;
      s_ok[t] = id >= 0;
      s_scl[t] = scl;
      s_mul[t] = sm_log2 * scl;
    }
    __syncthreads();
    if (s + 1 < nwork) gather(s + 1, cur);  // the next rows load meanwhile

    // S^T tiles: tokens tt*16 + (0..15) x the wave's 16 heads.
    f32x4_t sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint8_t* arow = lds_c + (tt * 16 + col) * kRowBytes + grp * 16;
      sacc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint4 av[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) av[kk] = *(const uint4*)(arow + (half * 8 + kk) * 64);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          sacc[tt] = mfma16x16x32(as_bf16x8(av[kk]), qb[half * 8 + kk], sacc[tt]);
      }
    }
    // lane holds S^T[token tt*16 + grp*4 + i][head col]
    float x[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = tt * 16 + grp * 4 + i;
        const float v = s_ok[tk] ? sacc[tt][i] * s_mul[tk] : -INFINITY;
        x[tt * 4 + i] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    // Lazy rescaling: a head's reference max m_run moves only when this
    // sub-chunk's max exceeds it by more than 8 (log2 units), so P stays below
    // 2^8 and O is rescaled only on the rare step that moves a reference.
    const bool move = mloc > m_run + 8.f;
    if (__any(move)) {
      const float alpha = move ? exp2f(m_run - mloc) : 1.f;  // exp2(-inf) = 0
      const bool live = __any(move && m_run != -INFINITY);     // O holds data to rescale
      if (move) m_run = mloc;
      l_run *= alpha;
      if (live) {
        float ai[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, grp * 4 + i, kWave);
#pragma unroll
        for (int G = 0; G < 4; ++G)
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[G][e][i] *= ai[i];
      }
    }
    const bool none = m_run == -INFINITY;
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = none ? 0.f : exp2f(x[k] - m_run);
      psum += p[k];
    }
    psum += __shfl_xor(psum, 16, kWave);
    psum += __shfl_xor(psum, 32, kWave);
    l_run += psum;

    // P as the A operand of O = P C: lane holds P[head col][K = grp*8 + k].
    uint32_t pw[4];
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      float p0 = p[k], p1 = p[k + 1];
      if (FP8) {
        const int t0 = (k < 4 ? 0 : 16) + grp * 4 + (k & 3);
        p0 *= s_scl[t0];
        p1 *= s_scl[t0 + 1];
      }
      pw[k >> 1] = f32_to_bf16_rne(p0) | (f32_to_bf16_rne(p1) << 16);
    }
    const bf16x8_t pa = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));

    // B operands: token rows grp*4+0..3 and 16+grp*4+0..3 (K order), 8 dims
    // G*128 + 8*col .. +7 per 16-byte read.
    const uint8_t* r0 = lds_c + (grp * 4) * kRowBytes + col * 16;
    const uint8_t* r1 = lds_c + (16 + grp * 4) * kRowBytes + col * 16;
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      uint4 u[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u[j] = *(const uint4*)(r0 + j * kRowBytes + G * 256);
        u[4 + j] = *(const uint4*)(r1 + j * kRowBytes + G * 256);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint32_t bw[4];
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) {
          const uint32_t a0 = u4_word(u[2 * m2], wd), a1 = u4_word(u[2 * m2 + 1], wd);
          bw[m2] = (e & 1) ? hi_pair(a0, a1) : lo_pair(a0, a1);
        }
        o[G][e] = mfma16x16x32(pa, as_bf16x8(make_uint4(bw[0], bw[1], bw[2], bw[3])), o[G][e]);
      }
    }
  };
  for (int s = 0; s < nwork; ++s) step(s, pre0);

  float li[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) li[i] = __shfl(l_run, grp * 4 + i, kWave);
  if (nchunks == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + grp * 4 + i;
      if (h >= Hm) continue;
      const float inv = li[i] > 0.f ? 1.f / li[i] : 0.f;
      uint16_t* orow = out + ((int64_t)qx * Hm + h) * L + col * 8;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2)
          pk[e >> 1] = f32_to_bf16_rne(o[G][e][i] * inv) | (f32_to_bf16_rne(o[G][e + 1][i] * inv) << 16);
        *(uint4*)(orow + G * 128) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      }
    }
    if (lse && grp == 0 && hq < Hm)
      lse[(int64_t)qx * Hm + hq] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t pbase = ((int64_t)qx * nchunks + chunk) * Hm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + grp * 4 + i;
      if (h >= Hm) continue;
      float* prow = part_o + (pbase + h) * L + col * 8;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        float4* d4 = (float4*)(prow + G * 128);
        d4[0] = make_float4(o[G][0][i], o[G][1][i], o[G][2][i], o[G][3][i]);
        d4[1] = make_float4(o[G][4][i], o[G][5][i], o[G][6][i], o[G][7][i]);
      }
    }
    if (grp == 0 && hq < Hm) {
      part_ml[(pbase + hq) * 2] = m_run;
      part_ml[(pbase + hq) * 2 + 1] = l_run;
    }
  }
}

// Merge the per-chunk partials of one (query, head) in chunk order; a wave per
// head, 8 dims per lane, four heads per workgroup.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int nchunks, int Hm,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6), qx = blockIdx.y, lane = threadIdx.x & 63;
  if (h >= Hm) return;
  const int64_t b0 = (int64_t)qx * nchunks * Hm + h;
  float M = -INFINITY;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, part_ml[(b0 + (int64_t)c * Hm) * 2]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll 4
  for (int c = 0; c < nchunks; ++c) {
    const int64_t pc = b0 + (int64_t)c * Hm;
    const float m = part_ml[pc * 2], l = part_ml[pc * 2 + 1];
    const float4* src = (const float4*)(part_o + pc * L + lane * 8);
    const float4 u = src[0], v = src[1];
    const float wgt = (M == -INFINITY) ? 0.f : exp2f(m - M);
    lsum = fmaf(l, wgt, lsum);
    acc[0] = fmaf(wgt, u.x, acc[0]);
    acc[1] = fmaf(wgt, u.y, acc[1]);
    acc[2] = fmaf(wgt, u.z, acc[2]);
    acc[3] = fmaf(wgt, u.w, acc[3]);
    acc[4] = fmaf(wgt, v.x, acc[4]);
    acc[5] = fmaf(wgt, v.y, acc[5]);
    acc[6] = fmaf(wgt, v.z, acc[6]);
    acc[7] = fmaf(wgt, v.w, acc[7]);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint32_t pk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    pk[k] = f32_to_bf16_rne(acc[2 * k] * inv) | (f32_to_bf16_rne(acc[2 * k + 1] * inv) << 16);
  *(uint4*)(out + ((int64_t)qx * Hm + h) * L + lane * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (lse && lane == 0)
    lse[(int64_t)qx * Hm + h] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
}

}  // namespace

DSA_EXPORT size_t dsa_sparse_mla_decode_workspace_size(int Q, int Hm, int L_, int out_width,
                                                       int latent_dtype) {
  (void)latent_dtype;
  if (Q <= 0 || Hm <= 0 || out_width <= 0 || L_ != L) return 0;
  const Chunking ch = mla_chunking(Q, Hm, out_width);
  if (ch.nchunks <= 1) return 0;
  const size_t rows = (size_t)Q * ch.nchunks * Hm;
  return rows * L * sizeof(float) + rows * 2 * sizeof(float);
}

DSA_EXPORT dsa_status dsa_sparse_mla_decode(const uint16_t* q, const void* ckv,
                                            const float* ckv_scale, int latent_dtype,
                                            const int32_t* kv_off, const int32_t* q_req,
                                            const int32_t* tok, int Q, int Hm, int L_,
                                            int out_width, float sm_scale, uint16_t* out,
                                            float* lse, void* ws, size_t ws_bytes,
                                            hipStream_t stream) {
  DSA_REQUIRE(L_ == L, DSA_ERR_UNSUPPORTED,
              "dsa_sparse_mla_decode: latent width L=%d, the kernels read exactly %d (a NoPE "
              "cache row is kv_lora_rank wide)",
              L_, L);
  DSA_REQUIRE(Hm >= 1, DSA_ERR_INVALID_ARG, "dsa_sparse_mla_decode: Hm=%d < 1 (no heads)", Hm);
  DSA_REQUIRE(out_width >= 1, DSA_ERR_INVALID_ARG, "dsa_sparse_mla_decode: out_width=%d < 1",
              out_width);
  DSA_REQUIRE(Q >= 0, DSA_ERR_INVALID_ARG, "dsa_sparse_mla_decode: Q=%d < 0", Q);
  DSA_REQUIRE(latent_dtype == DSA_LATENT_BF16 || latent_dtype == DSA_LATENT_FP8_E4M3,
              DSA_ERR_INVALID_ARG, "dsa_sparse_mla_decode: unknown latent dtype %d",
              latent_dtype);
  DSA_REQUIRE(latent_dtype != DSA_LATENT_FP8_E4M3 || ckv_scale, DSA_ERR_INVALID_ARG,
              "dsa_sparse_mla_decode: fp8 latent without row scales");
  if (Q == 0) return DSA_OK;
  DSA_REQUIRE(q && ckv && kv_off && q_req && tok && out, DSA_ERR_INVALID_ARG,
              "dsa_sparse_mla_decode: NULL tensor pointer");
  const size_t need = dsa_sparse_mla_decode_workspace_size(Q, Hm, L_, out_width, latent_dtype);
  DSA_REQUIRE(ws_bytes >= need && (need == 0 || ws), DSA_ERR_INVALID_ARG,
              "dsa_sparse_mla_decode: workspace %zu bytes, need %zu", ws_bytes, need);
  const Chunking ch = mla_chunking(Q, Hm, out_width);
  float* part_o = need ? (float*)ws : nullptr;
  float* part_ml = need ? (float*)ws + (size_t)Q * ch.nchunks * Hm * L : nullptr;
  dim3 grid(ch.nchunks, (Hm + 63) / 64, Q);
  const float sm_log2 = sm_scale * kLog2e;
  if (dsa::trace_enabled())
    fprintf(stderr, "[dsa] sparse_mla Q=%d Hm=%d out_width=%d fp8=%d chunks=%d tch=%d\n", Q, Hm,
            out_width, latent_dtype, ch.nchunks, ch.tch);
  if (latent_dtype == DSA_LATENT_FP8_E4M3)
    sparse_mla_kernel<true><<<grid, 256, 0, stream>>>(q, ckv, ckv_scale, kv_off, q_req, tok, Hm,
                                                      out_width, ch.tch, sm_log2, out, lse,
                                                      part_o, part_ml);
  else
    sparse_mla_kernel<false><<<grid, 256, 0, stream>>>(q, ckv, ckv_scale, kv_off, q_req, tok, Hm,
                                                       out_width, ch.tch, sm_log2, out, lse,
                                                       part_o, part_ml);
  dsa_status st = dsa::check_launch("dsa_sparse_mla_decode");
  if (st != DSA_OK || ch.nchunks == 1) return st;
  mla_combine_kernel<<<dim3((Hm + 3) / 4, Q), 256, 0, stream>>>(part_o, part_ml, ch.nchunks, Hm, out, lse);
  return dsa::check_launch("dsa_sparse_mla_decode (combine)");
}
