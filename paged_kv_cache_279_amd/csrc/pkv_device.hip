// Device side of libpkv: paged KV append, paged decode attention (partition
// kernel + log-sum-exp reduce kernel) for gfx950, and their C-ABI launchers.
//
// What is computed follows pgsm §4.2 (a decode step reads every cached K/V of
// the sequence, scores it against the query, normalises with a softmax and
// takes the weighted sum of the values) over the page-table store of
// hotelren §3.2 / pgsm §3.2, with in-place append (pgsm §4.3). The pages also
// say that reading the KV dominates a decode step (pgsm §4.2, dpshk §2.2), so
// every kernel here is organised around streaming the pool from HBM once.
//
// Decode kernel organisation (one workgroup = 4 waves per (sequence, KV head,
// partition)):
//   * a wave owns 16-token blocks blk = wave, wave + 4, ... of the partition;
//     each block is one contiguous 16 x D fp16 run inside a page tile, read
//     with fully coalesced 16-byte loads (lane l reads bytes 16 l .. 16 l + 15
//     of each 1 KiB slice), the next block's loads issued before the current
//     block is consumed;
//   * a lane holds 8 dims of NL tokens (D = 128: 16 lanes per token, 4 tokens
//     per load; D = 64: 8 lanes, 8 tokens); all G = Hq / Hkv query heads of the
//     group are served from the same K/V registers, so each K/V byte is read
//     from memory once per step;
//   * q.k uses v_dot2_f32_f16 (fp16 products, fp32 accumulation) and a DPP
//     reduction inside the lane group; the softmax is online (running max and
//     sum per lane group, fp32, base-2 exponent with the scale folded in);
//   * at the end the lane groups of a wave merge through cross-lane shuffles
//     and the 4 waves through LDS; the result is either the final fp16 row or
//     a (max, sum, unnormalised output) partial for the reduce kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBlk = 16;                   // tokens per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr size_t kWsAlign = 256;

struct DecodeParams {
  half_t* out;               // [B][Hq][D]
  const half_t* q;           // [B][Hq][D]
  const half_t* k_pool;      // [N][Hkv][P][D]
  const half_t* v_pool;
  half_t* k_pool_w;          // same pools, written by the fused append
  half_t* v_pool_w;
  const half_t* k_new;       // [B][Hkv][D] (fused append only)
  const half_t* v_new;
  const int32_t* bt;         // [B][max_pages]
  const int32_t* lens;       // [B]
  float* part_m;             // [B][Hq][n_parts], base-2 scaled score max
  float* part_l;             // [B][Hq][n_parts]
  float* part_o;             // [B][Hq][n_parts][D], unnormalised
  int32_t max_pages;
  int32_t B, Hq, Hkv, N;
  int32_t p_shift;           // log2(P)
  int32_t max_context;
  int32_t part_tokens;       // multiple of 16
  int32_t n_parts;           // partitions per sequence in this launch
  float scale_log2;          // scale * log2(e)
};

__device__ __forceinline__ float kNegInf() { return -__builtin_huge_valf(); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes that hold one token (LPT = 16 or 8);
// every lane of the group receives the total.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPT == 16) {
    x += dpp<0x128>(x);   // row_ror:8
    x += dpp<0x124>(x);   // row_ror:4
  } else {
    static_assert(LPT == 8, "lanes per token must be 8 or 16");
    x += dpp<0x141>(x);   // row_half_mirror
  }
  x += dpp<0x4E>(x);      // quad_perm [2,3,0,1]
  x += dpp<0xB1>(x);      // quad_perm [1,0,3,2]
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ __forceinline__ void unpack8(const uint4& v, float f[8]) {
  const half2_t a = as_h2(v.x), b = as_h2(v.y), c = as_h2(v.z), d = as_h2(v.w);
  f[0] = (float)a.x; f[1] = (float)a.y; f[2] = (float)b.x; f[3] = (float)b.y;
  f[4] = (float)c.x; f[5] = (float)c.y; f[6] = (float)d.x; f[7] = (float)d.y;
}

// -------------------------------------------------------------------------
// append
// -------------------------------------------------------------------------

// One thread per 16-byte chunk of (b, kvh, d/8): copies the new token's K and
// V chunk into slot (bt[b][pos/P], kvh, pos % P).
__global__ __launch_bounds__(256) void kv_append_kernel(const uint4* __restrict__ k_new,
                                                        const uint4* __restrict__ v_new,
                                                        uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                        const int32_t* __restrict__ bt, int32_t max_pages,
                                                        const int32_t* __restrict__ pos, int32_t B, int32_t Hkv,
                                                        int32_t d8, int32_t p_shift, int32_t N) {
  const int32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * Hkv * d8) return;
  const int32_t c = idx % d8;
  const int32_t r = idx / d8;
  const int32_t kvh = r % Hkv;
  const int32_t b = r / Hkv;
  const int32_t t = pos[b];
  if (t < 0 || (t >> p_shift) >= max_pages) return;
  const int32_t page = bt[(int64_t)b * max_pages + (t >> p_shift)];
  if (page < 0 || page >= N) return;
  const int64_t slot = ((((int64_t)page * Hkv + kvh) << p_shift) + (t & ((1 << p_shift) - 1))) * d8 + c;
  k_pool[slot] = k_new[idx];
  v_pool[slot] = v_new[idx];
}

// -------------------------------------------------------------------------
// decode: partition kernel
// -------------------------------------------------------------------------

template <int D, int G, bool SPLIT, bool FUSED>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeParams p) {
  constexpr int LPT = D / 8;           // lanes per token
  constexpr int TPI = kWave / LPT;     // tokens per 16-byte-per-lane load
  constexpr int NL = kBlk / TPI;       // loads per pool per block

  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];

  const int32_t id = blockIdx.x;
  const int32_t kvh = id % p.Hkv;      // consecutive ids -> consecutive KV heads (XCD round robin)
  const int32_t rest = id / p.Hkv;
  const int32_t b = rest % p.B;
  const int32_t part = rest / p.B;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane / LPT;
  const int dc = lane % LPT;

  const int32_t L = p.lens[b];
  const bool bad_len = L < 0 || L > p.max_context || L > (p.max_pages << p.p_shift);
  const int32_t Lc = bad_len ? 0 : L;
  const int32_t start = part * p.part_tokens;
  const int32_t end = min(Lc, start + p.part_tokens);
  const int64_t head_row0 = (int64_t)b * p.Hq + (int64_t)kvh * G;   // first query head of the group

  if (start >= end) {
    // nothing to attend in this partition; the unsplit kernel still owns the output row
    if (!SPLIT && part == 0) {
      const half_t fill = bad_len ? (half_t)__builtin_nanf("") : (half_t)0.0f;
      for (int i = threadIdx.x; i < G * D; i += kThreads) p.out[head_row0 * D + i] = fill;
    }
    return;
  }

  const int32_t* bt_row = p.bt + (int64_t)b * p.max_pages;
  const int32_t pmask = (1 << p.p_shift) - 1;
  const int64_t tile_elems = (int64_t)D << p.p_shift;       // one (page, kvh) tile

  // fused append: the workgroup owning the new token writes it to the pool
  uint4 knew = {0, 0, 0, 0}, vnew = {0, 0, 0, 0};
  const bool owns_new = FUSED && (start <= Lc - 1) && (Lc - 1 < end);
  if constexpr (FUSED) {
    if (owns_new) {
      const int64_t src = (((int64_t)b * p.Hkv + kvh) * D) / 8 + dc;
      knew = reinterpret_cast<const uint4*>(p.k_new)[src];
      vnew = reinterpret_cast<const uint4*>(p.v_new)[src];
      const int32_t t = Lc - 1;
      const int32_t page = bt_row[t >> p.p_shift];
      if (wave == 0 && grp == 0 && page >= 0 && page < p.N) {
        const int64_t dst = ((int64_t)page * p.Hkv + kvh) * tile_elems + (int64_t)(t & pmask) * D + dc * 8;
        *reinterpret_cast<uint4*>(p.k_pool_w + dst) = knew;
        *reinterpret_cast<uint4*>(p.v_pool_w + dst) = vnew;
      }
    }
  }

  // the group's query rows, 8 dims per lane, kept as packed fp16 pairs
  half2_t qv[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = *reinterpret_cast<const uint4*>(p.q + (head_row0 + h) * D + dc * 8);
    qv[h][0] = as_h2(t.x); qv[h][1] = as_h2(t.y); qv[h][2] = as_h2(t.z); qv[h][3] = as_h2(t.w);
  }

  float o[G][8];
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  bool bad_page = false;
  const float c = p.scale_log2;

  const int32_t nblocks = (end - start + kBlk - 1) / kBlk;

  auto tile_offset = [&](int32_t blk) -> int64_t {
    const int32_t t0 = start + blk * kBlk;
    int32_t page = bt_row[t0 >> p.p_shift];
    if (page < 0 || page >= p.N) {
      bad_page = true;
      page = 0;                         // stay in bounds; the row becomes NaN below
    }
    return ((int64_t)page * p.Hkv + kvh) * tile_elems + (int64_t)(t0 & pmask) * D;
  };

  auto load_block = [&](int32_t blk, uint4 kr[NL], uint4 vr[NL]) {
    const int64_t off = tile_offset(blk);
    const uint4* kp = reinterpret_cast<const uint4*>(p.k_pool + off) + lane;
    const uint4* vp = reinterpret_cast<const uint4*>(p.v_pool + off) + lane;
#pragma unroll
    for (int j = 0; j < NL; ++j) kr[j] = kp[j * kWave];
#pragma unroll
    for (int j = 0; j < NL; ++j) vr[j] = vp[j * kWave];
  };

  auto consume = [&](int32_t blk, uint4 kr[NL], uint4 vr[NL]) {
    const int32_t t0 = start + blk * kBlk;
    const bool tail = t0 + kBlk >= end;        // last block of the partition: mask / substitute
    if (tail) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int32_t tok = t0 + j * TPI + grp;
        if (FUSED && owns_new && tok == Lc - 1) {
          kr[j] = knew;
          vr[j] = vnew;
        }
        if (tok >= end) vr[j] = uint4{0, 0, 0, 0};     // never multiply unowned slots
      }
    }
    float s[NL][G];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
        acc = __builtin_amdgcn_fdot2(qv[h][0], as_h2(kr[j].x), acc, false);
        acc = __builtin_amdgcn_fdot2(qv[h][1], as_h2(kr[j].y), acc, false);
        acc = __builtin_amdgcn_fdot2(qv[h][2], as_h2(kr[j].z), acc, false);
        acc = __builtin_amdgcn_fdot2(qv[h][3], as_h2(kr[j].w), acc, false);
        s[j][h] = group_sum<LPT>(acc);
      }
    }
    if (tail) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int32_t tok = t0 + j * TPI + grp;
#pragma unroll
        for (int h = 0; h < G; ++h) s[j][h] = tok < end ? s[j][h] : kNegInf();
      }
    }
    float vf[NL][8];
#pragma unroll
    for (int j = 0; j < NL; ++j) unpack8(vr[j], vf[j]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = s[0][h];
#pragma unroll
      for (int j = 1; j < NL; ++j) bm = fmaxf(bm, s[j][h]);
      const float mn = fmaxf(m[h], bm * c);
      const float ms = mn == kNegInf() ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - ms);
      float pj[NL];
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        pj[j] = fast_exp2(fmaf(s[j][h], c, -ms));
        ps += pj[j];
      }
      l[h] = fmaf(l[h], alpha, ps);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = o[h][e] * alpha;
#pragma unroll
        for (int j = 0; j < NL; ++j) acc = fmaf(pj[j], vf[j][e], acc);
        o[h][e] = acc;
      }
      m[h] = mn;
    }
  };

  // software pipeline: next block's loads are in flight while this one is consumed
  uint4 ka[NL], va[NL], kb[NL], vb[NL];
  int32_t blk = wave;
  if (blk < nblocks) load_block(blk, ka, va);
  while (blk < nblocks) {
    const int32_t nxt = blk + kWaves;
    if (nxt < nblocks) load_block(nxt, kb, vb);
    consume(blk, ka, va);
    blk = nxt;
    if (blk >= nblocks) break;
    const int32_t nxt2 = blk + kWaves;
    if (nxt2 < nblocks) load_block(nxt2, ka, va);
    consume(blk, kb, vb);
    blk = nxt2;
  }

  // merge the lane groups of this wave (they saw disjoint tokens)
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float ms = mn == kNegInf() ? 0.f : mn;
      const float wa = fast_exp2(m[h] - ms);
      const float wb = fast_exp2(mo - ms);
      l[h] = l[h] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = o[h][e] * wa + __shfl_xor(o[h][e], off) * wb;
      m[h] = mn;
    }
  }
  if (bad_page) {
#pragma unroll
    for (int h = 0; h < G; ++h) l[h] = __builtin_nanf("");
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][h][dc * 8 + e] = o[h][e];
      if (dc == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // merge the waves and write
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    const float Ms = M == kNegInf() ? 0.f : M;
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][h] - Ms);
      Ls = fmaf(wt, sm_l[w][h], Ls);
      O = fmaf(wt, sm_o[w][h][d], O);
    }
    if constexpr (SPLIT) {
      const int64_t slot = (head_row0 + h) * p.n_parts + part;
      p.part_o[slot * D + d] = O;
      if (d == 0) {
        p.part_m[slot] = M;
        p.part_l[slot] = Ls;
      }
    } else {
      const float r = Ls > 0.f ? O / Ls : (Ls == 0.f ? 0.f : __builtin_nanf(""));
      p.out[(head_row0 + h) * D + d] = (half_t)(Ls != Ls ? __builtin_nanf("") : r);
    }
  }
}

// -------------------------------------------------------------------------
// decode: log-sum-exp reduce over partitions
// -------------------------------------------------------------------------

// One workgroup of D threads per (sequence, query head); thread d merges
// output dim d over the sequence's ceil(L / part_tokens) partitions.
template <int D>
__global__ __launch_bounds__(D) void lse_reduce_kernel(DecodeParams p) {
  const int64_t bh = blockIdx.x;
  const int32_t b = (int32_t)(bh / p.Hq);
  const int d = threadIdx.x;
  const int32_t L = p.lens[b];
  const bool bad_len = L < 0 || L > p.max_context || L > (p.max_pages << p.p_shift);
  const int32_t np = bad_len ? 0 : (L + p.part_tokens - 1) / p.part_tokens;
  const float* pm = p.part_m + bh * p.n_parts;
  const float* pl = p.part_l + bh * p.n_parts;
  const float* po = p.part_o + bh * p.n_parts * D + d;
  float M = kNegInf();
  for (int32_t j = 0; j < np; ++j) M = fmaxf(M, pm[j]);
  const float Ms = M == kNegInf() ? 0.f : M;
  float Ls = 0.f, O = 0.f;
  for (int32_t j = 0; j < np; ++j) {
    const float wt = fast_exp2(pm[j] - Ms);
    Ls = fmaf(wt, pl[j], Ls);
    O = fmaf(wt, po[(int64_t)j * D], O);
  }
  float r = Ls > 0.f ? O / Ls : 0.f;
  if (bad_len || Ls != Ls) r = __builtin_nanf("");
  p.out[bh * D + d] = (half_t)r;
}

// -------------------------------------------------------------------------
// host side
// -------------------------------------------------------------------------

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int log2_page(int32_t P) {
  switch (P) {
    case 16: return 4;
    case 32: return 5;
    case 64: return 6;
    case 128: return 7;
    default: return -1;
  }
}

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct WsLayout {
  size_t m_off, l_off, o_off, total;
};

WsLayout ws_layout(int64_t B, int64_t Hq, int64_t D, int64_t n_parts) {
  const size_t stats = align_up(static_cast<size_t>(B * Hq * n_parts) * sizeof(float));
  const size_t outs = align_up(static_cast<size_t>(B * Hq * n_parts * D) * sizeof(float));
  return WsLayout{0, stats, 2 * stats, 2 * stats + outs};
}

int32_t parts_for(int32_t max_context, int32_t partition_tokens) {
  return partition_tokens > 0 ? (max_context + partition_tokens - 1) / partition_tokens : 1;
}

template <int D, int G, bool SPLIT, bool FUSED>
hipError_t launch_partition(const DecodeParams& p, hipStream_t stream, int64_t grid) {
  hipLaunchKernelGGL((decode_partition_kernel<D, G, SPLIT, FUSED>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool SPLIT, bool FUSED>
hipError_t dispatch_g(int G, const DecodeParams& p, hipStream_t s, int64_t grid) {
  switch (G) {
    case 1: return launch_partition<D, 1, SPLIT, FUSED>(p, s, grid);
    case 2: return launch_partition<D, 2, SPLIT, FUSED>(p, s, grid);
    case 4: return launch_partition<D, 4, SPLIT, FUSED>(p, s, grid);
    default: return launch_partition<D, 8, SPLIT, FUSED>(p, s, grid);
  }
}

template <bool SPLIT, bool FUSED>
hipError_t dispatch_d(int D, int G, const DecodeParams& p, hipStream_t s, int64_t grid) {
  return D == 64 ? dispatch_g<64, SPLIT, FUSED>(G, p, s, grid) : dispatch_g<128, SPLIT, FUSED>(G, p, s, grid);
}

int decode_common(void* out, const void* q, const void* k_new, const void* v_new, const void* k_pool,
                  const void* v_pool, void* k_pool_w, void* v_pool_w, const int32_t* bt, int32_t max_pages,
                  const int32_t* lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                  int32_t max_context, float scale, int32_t partition_tokens, void* workspace,
                  size_t workspace_bytes, void* stream, bool fused) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || N <= 0 || max_pages <= 0 || max_context < 0 ||
      partition_tokens < 0)
    return PKV_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return PKV_ERR_INVALID_ARG;
  if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
    return PKV_ERR_INVALID_ARG;
  const int G = Hq / Hkv;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  const int p_shift = log2_page(P);
  if (p_shift < 0) return PKV_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PKV_ERR_UNSUPPORTED;
  if (partition_tokens % kBlk != 0) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_context) > (static_cast<int64_t>(max_pages) << p_shift)) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !bt || !lens) return PKV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(bt, 4) ||
      !aligned(lens, 4))
    return PKV_ERR_INVALID_ARG;
  if (fused && (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))) return PKV_ERR_INVALID_ARG;
  // every index the kernels form must fit in 64-bit arithmetic and the grid in 31 bits
  const int64_t pool_elems = static_cast<int64_t>(N) * Hkv * P * D;
  if (pool_elems / N / Hkv / P != D) return PKV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * max_pages > (int64_t{1} << 40)) return PKV_ERR_INVALID_ARG;

  const bool split = partition_tokens > 0;
  const int32_t n_parts = parts_for(max_context, partition_tokens);
  const int64_t grid = static_cast<int64_t>(n_parts) * B * Hkv;
  if (grid > 0x7fffffffLL || static_cast<int64_t>(B) * Hq > 0x7fffffffLL) return PKV_ERR_INVALID_ARG;

  DecodeParams prm{};
  prm.out = static_cast<half_t*>(out);
  prm.q = static_cast<const half_t*>(q);
  prm.k_pool = static_cast<const half_t*>(k_pool);
  prm.v_pool = static_cast<const half_t*>(v_pool);
  prm.k_pool_w = static_cast<half_t*>(k_pool_w);
  prm.v_pool_w = static_cast<half_t*>(v_pool_w);
  prm.k_new = static_cast<const half_t*>(k_new);
  prm.v_new = static_cast<const half_t*>(v_new);
  prm.bt = bt;
  prm.lens = lens;
  prm.max_pages = max_pages;
  prm.B = B;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.N = N;
  prm.p_shift = p_shift;
  prm.max_context = max_context;
  // unsplit: one partition covering any admissible length
  prm.part_tokens = split ? partition_tokens : ((max_context + kBlk - 1) / kBlk) * kBlk + kBlk;
  prm.n_parts = n_parts;
  prm.scale_log2 = scale * kLog2e;

  if (split) {
    const WsLayout ws = ws_layout(B, Hq, D, n_parts);
    if (!workspace) return PKV_ERR_INVALID_ARG;
    if (!aligned(workspace, kWsAlign)) return PKV_ERR_INVALID_ARG;
    if (workspace_bytes < ws.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
    char* base = static_cast<char*>(workspace);
    prm.part_m = reinterpret_cast<float*>(base + ws.m_off);
    prm.part_l = reinterpret_cast<float*>(base + ws.l_off);
    prm.part_o = reinterpret_cast<float*>(base + ws.o_off);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (grid > 0) {
    if (split) e = fused ? dispatch_d<true, true>(D, G, prm, s, grid) : dispatch_d<true, false>(D, G, prm, s, grid);
    else e = fused ? dispatch_d<false, true>(D, G, prm, s, grid) : dispatch_d<false, false>(D, G, prm, s, grid);
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  if (split) {
    const uint32_t rows = static_cast<uint32_t>(static_cast<int64_t>(B) * Hq);
    if (D == 64) hipLaunchKernelGGL(lse_reduce_kernel<64>, dim3(rows), dim3(64), 0, s, prm);
    else hipLaunchKernelGGL(lse_reduce_kernel<128>, dim3(rows), dim3(128), 0, s, prm);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* block_table,
                  int32_t max_pages, const int32_t* pos, int32_t B, int32_t Hkv, int32_t D, int32_t P, int32_t N,
                  void* stream) {
  if (B < 0 || Hkv <= 0 || D <= 0 || P <= 0 || N <= 0 || max_pages <= 0) return PKV_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  const int p_shift = log2_page(P);
  if (p_shift < 0) return PKV_ERR_UNSUPPORTED;
  if (B == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !pos) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_table, 4) || !aligned(pos, 4))
    return PKV_ERR_INVALID_ARG;
  const int64_t threads = static_cast<int64_t>(B) * Hkv * (D / 8);
  if (threads > 0x7fffffffLL) return PKV_ERR_INVALID_ARG;
  const int64_t pool_elems = static_cast<int64_t>(N) * Hkv * P * D;
  if (pool_elems / N / Hkv / P != D) return PKV_ERR_INVALID_ARG;
  const uint32_t blocks = static_cast<uint32_t>((threads + 255) / 256);
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), static_cast<uint4*>(k_pool),
                     static_cast<uint4*>(v_pool), block_table, max_pages, pos, B, Hkv, D / 8, p_shift, N);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_context, int32_t partition_tokens,
                               size_t* bytes) {
  if (!bytes || B < 0 || Hq <= 0 || D <= 0 || max_context < 0 || partition_tokens < 0 ||
      partition_tokens % kBlk != 0)
    return PKV_ERR_INVALID_ARG;
  *bytes = partition_tokens == 0 ? 0 : ws_layout(B, Hq, D, parts_for(max_context, partition_tokens)).total;
  return PKV_OK;
}

int pkv_paged_decode_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, int32_t max_pages, const int32_t* lens, int32_t B,
                               int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t N, int32_t max_context,
                               float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode_common(out, q, nullptr, nullptr, k_pool, v_pool, nullptr, nullptr, block_table, max_pages, lens, B,
                       Hq, Hkv, D, P, N, max_context, scale, partition_tokens, workspace, workspace_bytes, stream,
                       false);
}

int pkv_append_paged_decode_attention(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                      void* v_pool, const int32_t* block_table, int32_t max_pages,
                                      const int32_t* lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                                      int32_t N, int32_t max_context, float scale, int32_t partition_tokens,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(out, q, k_new, v_new, k_pool, v_pool, k_pool, v_pool, block_table, max_pages, lens, B, Hq,
                       Hkv, D, P, N, max_context, scale, partition_tokens, workspace, workspace_bytes, stream, true);
}

}  // extern "C"
