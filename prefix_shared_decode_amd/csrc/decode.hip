// Fused prefix-shared decode attention for gfx950 (MI355X).
//
// One launch runs a heterogeneous work list (BatchLLM summary, papercache.org,
// §5 "horizontal fusion"): each workgroup reads one item and runs either
//   * a mat-vec tile: one (query, kv head, KV chunk), the batched vector q
//     against paged K/V, memory bound (BatchLLM §2.1), or
//   * an MFMA prefix tile: every query row of one prefix-sharing group (and
//     kv head) stacked against one shared prefix chunk, so the prefix part is
//     a matrix multiply instead of a mat-vec (BatchLLM §2.2).
// Each tile produces a partial result (O, m, l) of its KV range; the tile
// that completes a (query, kv head) last merges all partials of it by online
// softmax (BatchLLM §2.2 Eq. 1) and writes the output, so no second launch is
// needed.
//
// Inside a tile scores live in log2 units (s * sm_scale * log2 e) so every
// exponential is one exp2; m is converted to natural-log units on output.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "psa_internal.h"

namespace psa {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.69314718055994531f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// weight of a partial with maximum m when merged into maximum M (log2 units)
__device__ __forceinline__ float rescale(float m, float M) { return m == -INFINITY ? 0.f : exp2f(m - M); }

// ---------------------------------------------------------------------------
// Output of one finished partial row (r heads x D) of query qi, kv head kvh.
// expected == 1: the tile owns the whole context and writes `out` directly;
// otherwise it stores the partial in its slot for the last arriver to merge.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_out(const DecodeParams& p, int64_t idx, float v) {
  if (p.out_bf16)
    reinterpret_cast<uint16_t*>(p.out)[idx] = f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(p.out)[idx] = v;
}

template <int D, int R>
__device__ __forceinline__ void store_row(const DecodeParams& p, int qi, int kvh, int hh, int slot_j, int dim0,
                                          const float* o, int n, bool write_ml, float m2, float l) {
  const int E = p.expected[qi];
  const int h = kvh * R + hh;
  if (E == 1) {
    const int64_t base = ((int64_t)qi * p.hq + h) * D + dim0;
    for (int e = 0; e < n; ++e) store_out(p, base + e, o[e]);
    if (write_ml) {
      if (p.out_m) p.out_m[(int64_t)qi * p.hq + h] = m2 * kLn2;
      if (p.out_l) p.out_l[(int64_t)qi * p.hq + h] = l;
    }
  } else {
    const int64_t S = ((int64_t)(p.slot_off[qi] + slot_j) * p.hkv + kvh) * R + hh;
    float* dst = p.part_o + S * D + dim0;
    for (int e = 0; e < n; ++e) dst[e] = o[e];
    if (write_ml) {
      p.part_ml[S * 2 + 0] = m2;
      p.part_ml[S * 2 + 1] = l;
    }
  }
}

// Merge all partials of (qi, kvh) in slot order and write the output; run by
// the whole workgroup.  Partials hold O normalised, m in log2 units, l.
template <int D, int R>
__device__ void merge_pair(const DecodeParams& p, int qi, int kvh) {
  const int E = p.expected[qi];
  const int64_t s0 = (int64_t)p.slot_off[qi];
  for (int el = threadIdx.x; el < R * D; el += kThreads) {
    const int hh = el / D, dim = el % D;
    float M = -INFINITY;
    for (int j = 0; j < E; ++j) {
      const int64_t S = ((s0 + j) * p.hkv + kvh) * R + hh;
      M = fmaxf(M, p.part_ml[S * 2]);
    }
    float L = 0.f, acc = 0.f;
    for (int j = 0; j < E; ++j) {
      const int64_t S = ((s0 + j) * p.hkv + kvh) * R + hh;
      const float w = p.part_ml[S * 2 + 1] * rescale(p.part_ml[S * 2], M);
      L += w;
      acc += w * p.part_o[S * D + dim];
    }
    const int h = kvh * R + hh;
    store_out(p, ((int64_t)qi * p.hq + h) * D + dim, L > 0.f ? acc / L : 0.f);
    if (dim == 0) {
      if (p.out_m) p.out_m[(int64_t)qi * p.hq + h] = L > 0.f ? M * kLn2 : -INFINITY;
      if (p.out_l) p.out_l[(int64_t)qi * p.hq + h] = L;
    }
  }
}

// Arrival: after every thread stored its partials, count one arrival for
// each listed query (kv head kvh) whose output needs a merge; the workgroup
// that brings a count to `expected` merges.  No waiting on other workgroups,
// so residency cannot deadlock; the fixed slot order of the merge makes the
// result independent of arrival order.
template <int D, int R>
__device__ void arrive(const DecodeParams& p, const int32_t* qlist, int nq, int kvh, int* s_last, int* s_nlast) {
  if (threadIdx.x == 0) *s_nlast = 0;
  __threadfence();  // release this thread's partial stores at agent scope
  __syncthreads();
  for (int t = threadIdx.x; t < nq; t += kThreads) {
    const int qi = qlist[t];
    const int E = p.expected[qi];
    if (E >= 2) {
      const int old = atomicAdd(&p.counters[(int64_t)qi * p.hkv + kvh], 1);
      if (old == E - 1) s_last[atomicAdd(s_nlast, 1)] = qi;
    }
  }
  __syncthreads();
  const int nl = *s_nlast;
  if (nl == 0) return;
  __threadfence();  // acquire: see every other tile's partials
  for (int t = 0; t < nl; ++t) merge_pair<D, R>(p, s_last[t], kvh);
  __syncthreads();
  for (int t = threadIdx.x; t < nl; t += kThreads) p.counters[(int64_t)s_last[t] * p.hkv + kvh] = 0;
}

// ---------------------------------------------------------------------------
// Mat-vec tile: one (query, kv head, token chunk).  A wave loads whole pages
// with 16-byte loads; LPT consecutive lanes hold one token's head_dim, so one
// load instruction reads TPW consecutive tokens = 1 KB contiguous of the page
// (pages are [kv head][16 tokens][D], one contiguous run per kv head).  All R
// query heads of the kv head are served by the same page read.  The 4 waves
// take pages round-robin; lane groups and waves merge their online-softmax
// states at the end.
// ---------------------------------------------------------------------------
template <int D, int R, bool BF16>
struct MatvecShape {
  static constexpr int EPL = BF16 ? 8 : 4;  // elements per 16-byte load
  static constexpr int LPT = D / EPL;       // lanes per token
  static constexpr int TPW = 64 / LPT;      // tokens per wave load
  static constexpr int LPP = 16 / TPW;      // loads per page per lane
};

template <int D, int R, bool BF16>
__device__ void matvec_tile(const DecodeParams& p, const WorkItem& it, char* smem) {
  using Sh = MatvecShape<D, R, BF16>;
  constexpr int EPL = Sh::EPL, LPT = Sh::LPT, TPW = Sh::TPW, LPP = Sh::LPP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qi = it.id, kvh = it.kvh;
  const int32_t* pages;
  if (it.kind == ITEM_MATVEC_DISTINCT) {
    pages = p.query_pages + p.query_page_off[qi];
  } else {
    const int g = p.query_group[qi];
    pages = p.group_pages + p.group_page_off[g];
  }
  const int tb = it.tok_begin, te = it.tok_end;
  const int pb = tb >> 4, pe = (te + 15) >> 4;
  const int dim0 = (lane % LPT) * EPL;
  const int tsub = lane / LPT;

  // query rows in registers
  u32x4 qv[R];
  {
    const int64_t qbase = ((int64_t)qi * p.hq + kvh * R) * D + dim0;
    for (int h = 0; h < R; ++h) {
      if constexpr (BF16)
        qv[h] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) + qbase + (int64_t)h * D);
      else
        qv[h] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(p.q) + qbase + (int64_t)h * D);
    }
  }
  float m[R], l[R], o[R][EPL];
  for (int h = 0; h < R; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }
  const float sc = p.scale_log2;
  const size_t elem = BF16 ? 2 : 4;
  const char* kbase = reinterpret_cast<const char*>(p.k);
  const char* vbase = reinterpret_cast<const char*>(p.v);

  auto load_page = [&](int pg, u32x4* kr, u32x4* vr) {
    const int64_t pid = pages[pg];
    const int64_t off = ((pid * p.hkv + kvh) * 16 + tsub) * D + dim0;
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int64_t o2 = (off + (int64_t)i * TPW * D) * elem;
      kr[i] = *reinterpret_cast<const u32x4*>(kbase + o2);
      vr[i] = *reinterpret_cast<const u32x4*>(vbase + o2);
    }
  };

  u32x4 kc[LPP], vc[LPP], kn[LPP], vn[LPP];
  int pg = pb + wave;
  if (pg < pe) load_page(pg, kc, vc);
  for (; pg < pe; pg += kWaves) {
    const int nxt = pg + kWaves;
    if (nxt < pe) load_page(nxt, kn, vn);
    // scores for this lane's LPP tokens, reduced over the LPT lanes of a token
    float s[LPP][R];
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
#pragma unroll
      for (int h = 0; h < R; ++h) {
        float acc = 0.f;
        if constexpr (BF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc = dot2_bf16(kc[i][w], qv[h][w], acc);
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(kc[i][w]), __uint_as_float(qv[h][w]), acc);
        }
        s[i][h] = acc;
      }
    }
#pragma unroll
    for (int off = LPT / 2; off >= 1; off >>= 1)
#pragma unroll
      for (int i = 0; i < LPP; ++i)
#pragma unroll
        for (int h = 0; h < R; ++h) s[i][h] += shfl_xor(s[i][h], off);
    const int tok0 = pg * 16 + tsub;
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < LPP; ++i) {
        s[i][h] = (tok0 + i * TPW < te) ? s[i][h] * sc : -INFINITY;
        mx = fmaxf(mx, s[i][h]);
      }
      const float mn = fmaxf(m[h], mx);
      if (mn == -INFINITY) continue;  // nothing valid yet in this lane group
      const float alpha = rescale(m[h], mn);
      m[h] = mn;
      float ps = 0.f;
      float pv[LPP];
#pragma unroll
      for (int i = 0; i < LPP; ++i) {
        pv[i] = exp2f(s[i][h] - mn);  // exp2(-inf) = 0 for masked tokens
        ps += pv[i];
      }
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < LPP; ++i) {
        if constexpr (BF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            o[h][2 * w] = fmaf(pv[i], bf16lo(vc[i][w]), o[h][2 * w]);
            o[h][2 * w + 1] = fmaf(pv[i], bf16hi(vc[i][w]), o[h][2 * w + 1]);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) o[h][w] = fmaf(pv[i], __uint_as_float(vc[i][w]), o[h][w]);
        }
      }
    }
    if (nxt < pe) {
#pragma unroll
      for (int i = 0; i < LPP; ++i) {
        kc[i] = kn[i];
        vc[i] = vn[i];
      }
    }
  }

  // merge the TPW lane groups of the wave (lanes with equal lane % LPT)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float mo = shfl_xor(m[h], off);
      const float lo = shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float a = rescale(m[h], mn), bw = rescale(mo, mn);
      l[h] = l[h] * a + lo * bw;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float oo = shfl_xor(o[h][e], off);
        o[h][e] = o[h][e] * a + oo * bw;
      }
      m[h] = mn;
    }
  }
  // merge the waves through LDS
  float* sm_m = reinterpret_cast<float*>(smem);          // [kWaves][R]
  float* sm_l = sm_m + kWaves * R;                        // [kWaves][R]
  float* sm_o = sm_l + kWaves * R;                        // [kWaves][R][D]
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[(wave * R + h) * D + dim0 + e] = o[h][e];
      if (lane == 0) {
        sm_m[wave * R + h] = m[h];
        sm_l[wave * R + h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int el = threadIdx.x; el < R * D; el += kThreads) {
    const int h = el / D, dim = el % D;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * R + h]);
    float L = 0.f, acc = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float a = rescale(sm_m[w * R + h], M);
      L += sm_l[w * R + h] * a;
      acc += sm_o[(w * R + h) * D + dim] * a;
    }
    const float ov = acc / L;  // every chunk holds >= 1 valid token, so L > 0
    store_row<D, R>(p, qi, kvh, h, it.slot, dim, &ov, 1, dim == 0, M, L);
  }
  __shared__ int32_t s_q[1];
  __shared__ int s_last[1];
  __shared__ int s_nlast;
  if (threadIdx.x == 0) s_q[0] = qi;
  __syncthreads();
  arrive<D, R>(p, s_q, 1, kvh, s_last, &s_nlast);
}

// ---------------------------------------------------------------------------
// MFMA prefix tile (bf16): rows = (member query, head in kv group) pairs of
// one group, up to 128 rows in 16-row slices (2 per wave), against one prefix
// chunk staged through LDS 64 tokens (4 pages) at a time.
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16: A = K rows (tokens), B = Q^T.
//   O^T = V^T P^T with the same MFMA:            A = V^T (from LDS), B = P^T.
// K rows are fed to the 16-row MFMA in the order token = 8*(m/4) + 4*half +
// m%4 (half = which of the two 16-token tiles of a 32-token block), so the
// S^T accumulator of lane group g holds 8 consecutive tokens of the block --
// exactly the k-slice lane group g supplies as the B operand (P^T) of the PV
// product.  P stays in registers; only V is transposed (when staged).
// ---------------------------------------------------------------------------
template <int D>
struct MfmaShape {
  static constexpr int KS = D + 8;   // K row stride in LDS (bf16)
  static constexpr int VS = 64 + 8;  // V^T row stride in LDS (bf16)
  static constexpr int KK = D / 32;  // k-steps of the QK product
  static constexpr int NB = D / 16;  // 16-wide dim blocks of O
  static constexpr int LDS_BYTES = (64 * KS + D * VS) * 2;
};

template <int D, int R>
__device__ void prefix_mfma_tile(const DecodeParams& p, const WorkItem& it, char* smem) {
  using Sh = MfmaShape<D>;
  constexpr int KS = Sh::KS, VS = Sh::VS, KK = Sh::KK, NB = Sh::NB;
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vt = Ks + 64 * KS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int g = it.id, kvh = it.kvh, rb = it.row_begin, rc = it.row_count;
  const int tb = it.tok_begin, te = it.tok_end;
  const int32_t* pages = p.group_pages + p.group_page_off[g];
  const int32_t* mem = p.members + p.member_off[g];
  const int nslices = (rc + 15) >> 4;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v);

  bool act[2];
  bf16x8 qb[2][KK];
  for (int sl = 0; sl < 2; ++sl) {
    const int slice = wave + kWaves * sl;
    const int row = slice * 16 + l16;
    act[sl] = slice < nslices;
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (act[sl] && row < rc) {
        const int grow = rb + row;
        const int qi = mem[grow / R];
        const int64_t off = ((int64_t)qi * p.hq + kvh * R + grow % R) * D + kk * 32 + lg * 8;
        w = *reinterpret_cast<const u32x4*>(qp + off);
      }
      qb[sl][kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  f32x4 oacc[2][NB];
  for (int sl = 0; sl < 2; ++sl)
    for (int nb = 0; nb < NB; ++nb) oacc[sl][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.f, 0.f};
  const float sc = p.scale_log2;
  constexpr int CPT = D / 8;                      // 16-byte chunks per token
  constexpr int LOADS = 64 * CPT / kThreads;      // per thread per stage

  for (int blk = tb; blk < te; blk += 64) {
    // ---- stage 64 tokens of K (row-major) and V (transposed) in LDS ----
    u32x4 kr[LOADS], vr[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = i * kThreads + tid;
      const int tok = idx / CPT, c = idx % CPT;
      const int t = blk + tok;
      kr[i] = u32x4{0u, 0u, 0u, 0u};
      vr[i] = u32x4{0u, 0u, 0u, 0u};
      if (t < te) {
        const int64_t off = (((int64_t)pages[t >> 4] * p.hkv + kvh) * 16 + (t & 15)) * D + c * 8;
        kr[i] = *reinterpret_cast<const u32x4*>(kp + off);
        vr[i] = *reinterpret_cast<const u32x4*>(vp + off);
      }
    }
    __syncthreads();  // previous stage fully consumed
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = i * kThreads + tid;
      const int tok = idx / CPT, c = idx % CPT;
      *reinterpret_cast<u32x4*>(Ks + tok * KS + c * 8) = kr[i];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        Vt[(c * 8 + 2 * w) * VS + tok] = (uint16_t)(vr[i][w] & 0xffffu);
        Vt[(c * 8 + 2 * w + 1) * VS + tok] = (uint16_t)(vr[i][w] >> 16);
      }
    }
    __syncthreads();
    if (!act[0]) continue;

    // ---- S^T tiles: t = kb*2 + half covers tokens 32kb + {8*(m/4) + 4*half + m%4} ----
    f32x4 st[2][4];
    for (int sl = 0; sl < 2; ++sl)
      for (int t = 0; t < 4; ++t) st[sl][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, half = t & 1;
      const int tokrow = kb * 32 + 8 * (l16 >> 2) + 4 * half + (l16 & 3);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + tokrow * KS + kk * 32 + lg * 8);
        st[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[0][kk], st[0][t], 0, 0, 0);
        if (act[1]) st[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[1][kk], st[1][t], 0, 0, 0);
      }
    }
    // ---- online softmax per row (lane's row = l16; 16 scores per lane) ----
    bf16x8 pb[2][2];
    for (int sl = 0; sl < 2; ++sl) {
      if (!act[sl]) continue;
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, half = t & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = blk + kb * 32 + 8 * lg + 4 * half + i;
          const float s = tok < te ? st[sl][t][i] * sc : -INFINITY;
          st[sl][t][i] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mn = fmaxf(mrow[sl], mx);  // finite: every block has a valid token
      const float alpha = rescale(mrow[sl], mn);
      mrow[sl] = mn;
      float ps = 0.f;
      float pr[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[t][i] = exp2f(st[sl][t][i] - mn);
          ps += pr[t][i];
        }
      lrow[sl] = lrow[sl] * alpha + ps;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[sl][nb] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = (__bf16)pr[kb * 2][i];
          v[4 + i] = (__bf16)pr[kb * 2 + 1][i];
        }
        pb[sl][kb] = v;
      }
    }
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vt + (nb * 16 + l16) * VS + kb * 32 + lg * 8);
        oacc[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[0][kb], oacc[0][nb], 0, 0, 0);
        if (act[1]) oacc[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[1][kb], oacc[1][nb], 0, 0, 0);
      }
    }
  }

  // ---- write each row's partial (or the output when the chunk is all of it) ----
  for (int sl = 0; sl < 2; ++sl) {
    if (!act[sl]) continue;
    float L = lrow[sl];
    L += shfl_xor(L, 16);
    L += shfl_xor(L, 32);
    const int row = (wave + kWaves * sl) * 16 + l16;
    if (row >= rc) continue;
    const int grow = rb + row;
    const int qi = mem[grow / R], hh = grow % R;
    const float inv = 1.f / L;
    for (int nb = 0; nb < NB; ++nb) {
      float ov[4];
      for (int i = 0; i < 4; ++i) ov[i] = oacc[sl][nb][i] * inv;
      store_row<D, R>(p, qi, kvh, hh, it.slot, nb * 16 + lg * 4, ov, 4, nb == 0 && lg == 0, mrow[sl], L);
    }
  }
  __shared__ int32_t s_q[128];
  __shared__ int s_last[128];
  __shared__ int s_nlast;
  const int nq = rc / R;
  for (int t = tid; t < nq; t += kThreads) s_q[t] = mem[rb / R + t];
  __syncthreads();
  arrive<D, R>(p, s_q, nq, kvh, s_last, &s_nlast);
}

// Empty partial (0, -inf, 0) of every head of a query whose context the plan
// does not cover (PREFIX_ONLY / DISTINCT_ONLY plans).
template <int D>
__device__ void empty_item(const DecodeParams& p, const WorkItem& it) {
  const int qi = it.id;
  for (int el = threadIdx.x; el < p.hq * D; el += kThreads) {
    store_out(p, (int64_t)qi * p.hq * D + el, 0.f);
    if (el % D == 0) {
      const int h = el / D;
      if (p.out_m) p.out_m[(int64_t)qi * p.hq + h] = -INFINITY;
      if (p.out_l) p.out_l[(int64_t)qi * p.hq + h] = 0.f;
    }
  }
}

template <int D, int R, bool BF16>
struct Lds {
  static constexpr int MV = (2 * kWaves * R + kWaves * R * D) * 4;
  static constexpr int MF = BF16 ? MfmaShape<D>::LDS_BYTES : 0;
  static constexpr int BYTES = MV > MF ? MV : MF;
};

template <int D, int R, bool BF16>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char smem[Lds<D, R, BF16>::BYTES];
  const WorkItem it = p.items[blockIdx.x];
  switch (it.kind) {
    case ITEM_MATVEC_DISTINCT:
    case ITEM_MATVEC_PREFIX:
      matvec_tile<D, R, BF16>(p, it, smem);
      break;
    case ITEM_PREFIX_MFMA:
      if constexpr (BF16) prefix_mfma_tile<D, R>(p, it, smem);
      break;
    case ITEM_EMPTY:
      empty_item<D>(p, it);
      break;
    default:
      break;
  }
}

template <int D, int R, bool BF16>
static hipError_t launch(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<D, R, BF16>), dim3(p.num_items), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_r(const DecodeParams& p, int r, hipStream_t s) {
  switch (r) {
    case 1: return launch<D, 1, BF16>(p, s);
    case 2: return launch<D, 2, BF16>(p, s);
    case 4: return launch<D, 4, BF16>(p, s);
    case 8: return launch<D, 8, BF16>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int head_dim, int r, bool bf16, hipStream_t s) {
  if (p.num_items <= 0) return hipSuccess;
  if (head_dim == 64) return bf16 ? launch_r<64, true>(p, r, s) : launch_r<64, false>(p, r, s);
  if (head_dim == 128) return bf16 ? launch_r<128, true>(p, r, s) : launch_r<128, false>(p, r, s);
  return hipErrorInvalidValue;
}

}  // namespace psa
