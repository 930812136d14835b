// Fused prefix-shared decode attention for gfx950 (MI355X).
//
// One launch runs a heterogeneous work list (BatchLLM summary, papercache.org,
// §5 "horizontal fusion"): each workgroup runs one unit, which is either
//   * an MFMA prefix tile: every query row of one prefix-sharing group (one
//     kv head, up to 128 rows) against one shared prefix chunk, so the prefix
//     part is a matrix multiply instead of a mat-vec (BatchLLM §2.2), or
//   * up to four mat-vec tiles, one per wave: one (query, kv head, KV chunk)
//     each, the batched vector q against paged K/V, memory bound (BatchLLM
//     §2.1).
// Each tile produces a partial result (O, m, l) of its KV range.  The tile
// that completes a (query, kv head) last merges all of its partials by online
// softmax (BatchLLM §2.2 Eq. 1) and writes the output, so no second launch is
// needed.  Partials travel through memory with device-coherent (sc1) stores
// and loads; ordering is a wait for store completion before the arrival
// counter's atomic add, so no L2 writeback or invalidate is ever issued.
//
// Scores live in log2 units (s * sm_scale * log2 e), so each exponential is a
// single v_exp_f32; m is converted to natural-log units on output.  Running
// maxima are "lazy": the reference max used for exponentials only moves when
// a score exceeds it by more than 8 (p <= 2^8), which makes rescaling of the
// accumulators rare; the true max is tracked alongside for the output.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "layout.h"
#include "psa_internal.h"

namespace psa {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNoMax = -1.0e30f;  // reference max of an empty state (finite: exp2 stays NaN-free)
constexpr int kNoLimit = 1 << 30;   // MFMA tile: row limit of a query that sees its whole prefix
constexpr float kLazy = 8.0f;       // MFMA tile: rescale only when a score exceeds the reference max by this
constexpr float kSlack = 16.0f;     // mat-vec tile: a fixed reference max may be exceeded by this much

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// ---------------------------------------------------------------- helpers ---
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// A wave-uniform float held in a scalar register (the value of the first active lane).
__device__ __forceinline__ float uniform_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Sum over the 8 consecutive lanes holding one token (lane % 8 varies):
// quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2), row_half_mirror.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v;
}
// Value of lane (i + 8) mod 16 within each row of 16 (row_ror:8) == lane i ^ 8.
__device__ __forceinline__ float xor8(float v) { return dpp<0x128>(v); }
// A lane's value and that of lane ^ OFF (OFF = 8, 16 or 32), in an order that
// depends on the lane; for symmetric combinations only.  8: row_ror:8 (DPP);
// 16: v_permlane16_swap (odd and even rows of 16); 32: v_permlane32_swap.
template <int OFF>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  if constexpr (OFF == 8) {
    a = v;
    b = xor8(v);
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    static_assert(OFF == 32, "lane distance 8, 16 or 32");
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

// Max over the four lanes l, l^16, l^32, l^48 (in the MFMA tile: the lane
// groups sharing one row): swap the 32-lane halves, then the odd and even
// 16-lane rows.
__device__ __forceinline__ float max_lane_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
#ifndef PSA_MV_PAGES
#define PSA_MV_PAGES 2
#endif
constexpr int kMvPages = PSA_MV_PAGES;  // mat-vec tile: bf16 pages of K and V in flight per wave
// (an fp32 page is twice the bytes: two of them with d 128 and R 8 do not fit
// the register budget, so that shape keeps one page in flight)
template <int D, int R, bool BF16>
constexpr int mv_pages() { return BF16 || D * R < 1024 ? kMvPages : 1; }
#ifndef PSA_MERGE_BATCH
#define PSA_MERGE_BATCH 8
#endif
constexpr int kMergeUnroll = PSA_MERGE_BATCH;  // merges of up to this many pieces load every piece in one pass
constexpr int kSc1 = 16;  // cache policy: coherent at device (agent) scope
constexpr int kNt = 2;    // cache policy: non-temporal (streamed once; keeps reused prefix K/V and
                          // partials from being evicted by the distinct KV stream)

__device__ __forceinline__ void st_coh4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kSc1);
}
__device__ __forceinline__ void st_coh1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4 ld_coh4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}
__device__ __forceinline__ float ld_coh1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1));
}

// Make this thread's partial stores complete (device-coherent) before what follows.
__device__ __forceinline__ void release_partials() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
}

__device__ __forceinline__ int arrive_counter(int32_t* c) {
  return __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(int32_t* c) {
  __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_out4(const DecodeParams& p, int64_t idx, f32x4 v) {
  if (p.out_bf16) {
    uint2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + idx) = w;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + idx) = v;
  }
}

__device__ __forceinline__ void store_ml(const DecodeParams& p, int64_t row, float m2, float l) {
  if (p.out_m) p.out_m[row] = l > 0.f ? m2 * kLn2 : -INFINITY;
  if (p.out_l) p.out_l[row] = l;
}

// Merge the E partials of (query qi, kv head kvh) in slot order and write the
// output; one wave.  Partials hold O normalised, m (log2 units), l.  No
// multiply-add is contracted here, so that the MFMA tile's merge in registers
// (same operations, same order) gives the same bits.  Lane l covers the
// float4 chunks l, l + 64, ... of the R x D rows.  Piece jown (if >= 0) is
// the calling wave's own, not written to memory: its O rows are at own_o in
// LDS (row-major, fp32), its m and l in own_m / own_l (the values its
// partial would have held, so the result does not depend on which piece
// merges).  With few pieces every load of every piece is issued at once.
template <int D, int R>
__device__ __forceinline__ void merge_pieces(const DecodeParams& p, int qi, int kvh, int E, int jown,
                                             const __attribute__((address_space(3))) float* own_o,
                                             const float (&own_m)[R], const float (&own_l)[R]) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int64_t s0 = p.slot_off[qi];
  const auto ro = make_rsrc(p.part_o, p.part_o_bytes);
  const auto rm = make_rsrc(p.part_ml, p.part_ml_bytes);
  constexpr int C4 = D / 4;                  // float4 chunks per row
  constexpr int NCI = (R * C4 + 63) / 64;    // chunks per lane
  int hh[NCI], c4[NCI];
  bool ok[NCI];
  float om[NCI], ol[NCI];  // the own piece's m and l for the lane's rows
#pragma unroll
  for (int k = 0; k < NCI; ++k) {
    const int ci = lane + 64 * k;
    ok[k] = ci < R * C4;
    hh[k] = ok[k] ? ci / C4 : 0;
    c4[k] = ci % C4;
    om[k] = own_m[0];
    ol[k] = own_l[0];
#pragma unroll
    for (int h = 1; h < R; ++h) {
      om[k] = hh[k] == h ? own_m[h] : om[k];
      ol[k] = hh[k] == h ? own_l[h] : ol[k];
    }
  }
  auto srow = [&](int j, int k) { return (uint32_t)(((s0 + j) * p.hkv + kvh) * R + hh[k]); };
  auto own4 = [&](int k) { return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(own_o + hh[k] * D + c4[k] * 4); };
  float M[NCI], L[NCI];
  f32x4 acc[NCI];
#pragma unroll
  for (int k = 0; k < NCI; ++k) {
    M[k] = kNoMax;
    L[k] = 0.f;
    acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (NCI <= 2 && E <= kMergeUnroll) {
    float mj[kMergeUnroll][NCI], lj[kMergeUnroll][NCI];
    f32x4 oj[kMergeUnroll][NCI];
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j)
#pragma unroll
      for (int k = 0; k < NCI; ++k) {
        mj[j][k] = om[k];
        lj[j][k] = ol[k];
        oj[j][k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j >= E) continue;
        if (j == jown) {
          oj[j][k] = own4(k);
        } else {
          mj[j][k] = ld_coh1(rm, srow(j, k) * 8u);
          lj[j][k] = ld_coh1(rm, srow(j, k) * 8u + 4u);
          oj[j][k] = ld_coh4(ro, (srow(j, k) * D + c4[k] * 4) * 4u);
        }
      }
#pragma unroll
    for (int k = 0; k < NCI; ++k) {
#pragma unroll
      for (int j = 0; j < kMergeUnroll; ++j)
        if (j < E) M[k] = fmaxf(M[k], mj[j][k]);
#pragma unroll
      for (int j = 0; j < kMergeUnroll; ++j) {
        if (j >= E) continue;
        const float w = lj[j][k] * fast_exp2(mj[j][k] - M[k]);
        L[k] += w;
        acc[k] += w * oj[j][k];
      }
    }
  } else {
#pragma unroll 2
    for (int j = 0; j < E; ++j)
#pragma unroll
      for (int k = 0; k < NCI; ++k) M[k] = fmaxf(M[k], j == jown ? om[k] : ld_coh1(rm, srow(j, k) * 8u));
#pragma unroll 2
    for (int j = 0; j < E; ++j)
#pragma unroll
      for (int k = 0; k < NCI; ++k) {
        if (j == jown) {
          const float w = ol[k] * fast_exp2(om[k] - M[k]);
          L[k] += w;
          acc[k] += w * own4(k);
        } else {
          const float w = ld_coh1(rm, srow(j, k) * 8u + 4u) * fast_exp2(ld_coh1(rm, srow(j, k) * 8u) - M[k]);
          L[k] += w;
          acc[k] += w * ld_coh4(ro, (srow(j, k) * D + c4[k] * 4) * 4u);
        }
      }
  }
#pragma unroll
  for (int k = 0; k < NCI; ++k) {
    if (!ok[k]) continue;
    const int64_t row = (int64_t)qi * p.hq + kvh * R + hh[k];
    store_out4(p, row * D + c4[k] * 4, acc[k] * (1.f / L[k]));
    if (c4[k] == 0) store_ml(p, row, M[k], L[k]);
  }
}

// The same merge with every piece in memory (the last arriving piece wrote
// its partial first).
template <int D, int R>
__device__ void merge_wave(const DecodeParams& p, int qi, int kvh) {
  const float none[R] = {};
  merge_pieces<D, R>(p, qi, kvh, p.expected[qi], -1, nullptr, none, none);
}

// ----------------------------------------------------------- mat-vec tile ---
// One wave, one (query, kv head, token chunk).  LPT consecutive lanes hold one
// token: lane c = lane % LPT covers the 16-byte chunks k*LPT + c of the
// token's row (k < NCH), so each load instruction reads 64/LPT whole tokens as
// contiguous runs; a page (16 tokens) is NT = LPT/4 token slots per lane.  All
// R query heads of the kv head share one read of the page.  Scores are summed
// over the LPT lanes with DPP; P.V uses bf16 dot2 over pairs of the lane's
// tokens.  LPT is 8 unless R * dims-per-lane would exceed 64 accumulators.
// The next page is in flight while one is computed; buffer loads use a descriptor covering the
// valid tokens of one (page, kv head) tile: a page past the chunk, and the slots past the
// chunk's end in its last page, read zeros with no traffic (so whatever those slots hold, NaN
// included, never meets a weight).  Pages are loaded non-temporal: each byte is read once.
// P is rounded to bf16 for the P.V dot products; O is normalised by the sum of those rounded
// weights (a convex combination of V rows), while the reported l is the exact fp32 sum.
// q is staged once through LDS (per wave); bf16 rows of up to 512 elements
// stay in registers for the page loop, larger ones are re-read per page.
template <int D, int R, bool BF16>
struct MvShape {
  static constexpr int EB = BF16 ? 2 : 4;
  static constexpr int CPT = D * EB / 16;       // 16-byte chunks per token row
  static constexpr int LPT = (R * (CPT / 8) * (16 / EB) > 64) ? 16 : 8;
  static constexpr int NCH = CPT / LPT;         // chunks per lane per token
  static constexpr int EPC = 16 / EB;           // elements per chunk
  static constexpr int DPL = NCH * EPC;         // dims per lane
  static constexpr int NT = 16 * LPT / 64;      // token slots per lane per page
  static constexpr int TSTEP = 64 / LPT;        // token distance between slots
  static constexpr uint32_t TILE = 16 * D * EB;
  static constexpr int QBYTES = R * D * EB;     // one wave's q rows in LDS
  // a wave's own fp32 O rows for a merge in registers: in its q rows' place
  // when they fit (fp32), else after all waves' q rows (a wave still reading
  // its q rows must not see them overwritten)
  static constexpr int OBYTES = R * D * 4;
  static constexpr int OWN_BASE = QBYTES >= OBYTES ? 0 : 4 * QBYTES;
  static constexpr int OWN_STRIDE = QBYTES >= OBYTES ? QBYTES : OBYTES;
  static constexpr int LDS_BYTES = OWN_BASE + 4 * OWN_STRIDE;  // for four waves
};

template <int D, int R, bool BF16>
struct PageRegs {
  u32x4 k[MvShape<D, R, BF16>::NT][MvShape<D, R, BF16>::NCH];
  u32x4 v[MvShape<D, R, BF16>::NT][MvShape<D, R, BF16>::NCH];
};

template <int LPT>
__device__ __forceinline__ float sum_lanes(float v) {
  v = sum8(v);
  if constexpr (LPT == 16) v += dpp<0x140>(v);  // row_mirror pairs the two half rows
  return v;
}

template <int D, int R, bool BF16>
__device__ __forceinline__ void matvec_wave(const DecodeParams& p, const WorkItem& it, char* smem) {
  using S = MvShape<D, R, BF16>;
  constexpr int NCH = S::NCH, EPC = S::EPC, DPL = S::DPL, LPT = S::LPT, NT = S::NT, TSTEP = S::TSTEP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % LPT, ts = lane / LPT;
  const int qi = it.id, kvh = it.kvh;
  const int tb = it.tok_begin, te = it.tok_end;
  const int npages = (te - tb + 15) >> 4;
  const uint32_t last_bytes = (uint32_t)(te - tb - 16 * (npages - 1)) * (D * S::EB);  // valid part of the last page
  const int pid_lane = lane < npages ? p.pages[it.page_base + lane] : 0;

  // stage this wave's q rows (R * D elements, contiguous) in LDS
  lds_char* qs = (lds_char*)(smem + wave * S::QBYTES);
  {
    const char* qg = reinterpret_cast<const char*>(p.q) + (((int64_t)qi * p.hq + kvh * R) * D) * S::EB;
    for (int o16 = lane; o16 < S::QBYTES / 16; o16 += 64)
      *(__attribute__((address_space(3))) u32x4*)(qs + o16 * 16) = *reinterpret_cast<const u32x4*>(qg + o16 * 16);
  }
  float mref[R], mtrue[R], l[R], lr[R], o[R][DPL];  // l: exact weights; lr: their bf16 roundings
  const float sc = p.scale_log2;
  const char* kpool = reinterpret_cast<const char*>(p.k);
  const char* vpool = reinterpret_cast<const char*>(p.v);

  auto load = [&](PageRegs<D, R, BF16>& b, int j) {
    // j beyond the chunk: an empty descriptor reads zeros without memory traffic
    const int pid = __builtin_amdgcn_readlane(pid_lane, j < npages ? j : 0);
    const int64_t tile = ((int64_t)pid * p.hkv + kvh) * S::TILE;
    const uint32_t bytes = j < npages - 1 ? S::TILE : (j == npages - 1 ? last_bytes : 0u);
    const auto rk = make_rsrc(kpool + tile, bytes);
    const auto rv = make_rsrc(vpool + tile, bytes);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const uint32_t off = (uint32_t)(((ts + TSTEP * t) * D + (k * LPT + c) * EPC) * S::EB);
        b.k[t][k] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kNt);
        b.v[t][k] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kNt);
      }
  };

  // Page j, one head at a time (so only NT scores are live): the scores (log2
  // units, masked tokens -inf); on the first page of the first pass, the
  // head's reference max; the exponentials against it; P.V.
  auto page = [&](const PageRegs<D, R, BF16>& b, int j, bool set_ref, bool& over) {
    // q from LDS: held in registers across the page loop where R * D <= 512
    // bf16 elements (32 VGPRs); re-read every page otherwise (an opaque
    // offset keeps the reads in the loop), where holding it would spill
    uint32_t qoff = (uint32_t)(c * EPC * S::EB);
    if constexpr (!(BF16 && R * D <= 512)) asm volatile("" : "+v"(qoff));
    const int tok0 = tb + j * 16 + ts;
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = 0.f;
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const u32x4 qv = *(const __attribute__((address_space(3))) u32x4*)(qs + qoff + (h * D + k * LPT * EPC) * S::EB);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (BF16)
              acc[t] = dot2_bf16(b.k[t][k][w], qv[w], acc[t]);
            else
              acc[t] = fmaf(__uint_as_float(b.k[t][k][w]), __uint_as_float(qv[w]), acc[t]);
          }
      }
      float sh[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sh[t] = tok0 + TSTEP * t < te ? sum_lanes<LPT>(acc[t]) * sc : -INFINITY;
      if (set_ref) {
        float mx = sh[0];
#pragma unroll
        for (int t = 1; t < NT; ++t) mx = fmaxf(mx, sh[t]);
        mx = fmaxf(mx, xor8(mx));
        mx = max_lane_groups(mx);  // page 0 always holds a valid token
        mref[h] = uniform_f(mx);   // the max over every token slot of the page: the same in each lane
        mtrue[h] = -INFINITY;
      }
      float pr[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        mtrue[h] = fmaxf(mtrue[h], sh[t]);
        over |= sh[t] > mref[h] + kSlack;
        pr[t] = fast_exp2(sh[t] - mref[h]);  // exp2(-inf) = 0 for masked tokens
        l[h] += pr[t];
      }
      if constexpr (BF16) {
#pragma unroll
        for (int t = 0; t < NT; t += 2) {
          const uint32_t pp = pack_bf16(pr[t], pr[t + 1]);
          lr[h] = dot2_bf16(pp, 0x3F803F80u, lr[h]);  // + the two rounded weights (times bf16 1.0)
#pragma unroll
          for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t a = b.v[t][k][w], bb = b.v[t + 1][k][w];
              o[h][k * 8 + 2 * w] = dot2_bf16(__builtin_amdgcn_perm(bb, a, 0x05040100u), pp, o[h][k * 8 + 2 * w]);
              o[h][k * 8 + 2 * w + 1] =
                  dot2_bf16(__builtin_amdgcn_perm(bb, a, 0x07060302u), pp, o[h][k * 8 + 2 * w + 1]);
            }
        }
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w) o[h][k * 4 + w] = fmaf(pr[t], __uint_as_float(b.v[t][k][w]), o[h][k * 4 + w]);
      }
    }
  };

  // The reference max is fixed per item (no rescaling inside the page loop):
  // the first page's wave-wide max per head.  A later score above it by more
  // than kSlack flags the item, which is then redone with the exact maximum
  // found by the first pass (so it cannot be exceeded).
  // The arrival counter of (query, kv head) is read while the last pages are
  // processed: if every other piece has arrived by then, this wave merges in
  // registers at the end instead of writing a partial.
  const int E = it.a, slot = it.b;
  int32_t* ctr = p.counters + (int64_t)qi * p.hkv + kvh;
  int cval = -1;
  bool ctr_read = E < 2;
  auto read_ctr = [&]() {
    cval = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ctr_read = true;
  };
  bool fixed_ref = false;
  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      l[h] = 0.f;
      lr[h] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
    }
    bool over = false;
    // a ring of NP page buffers: page j lives in buffer j % NP, and its load
    // is issued NP pages ahead of its use
    constexpr int NP = mv_pages<D, R, BF16>();
    PageRegs<D, R, BF16> b[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) load(b[u], u);
    page(b[0], 0, !fixed_ref, over);
    load(b[0], NP);
    for (int j = 1; j < npages; j += NP) {
      if (!ctr_read && j + NP >= npages) read_ctr();
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int bi = (u + 1) % NP;
        if (j + u < npages) page(b[bi], j + u, false, over);  // wave-uniform; loads past the end read zeros
        load(b[bi], j + u + NP);
      }
    }
    if (!ctr_read) read_ctr();
    if (!__builtin_amdgcn_ballot_w64(over)) break;
    // rare: redo with the exact per-head maximum of this chunk
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mx = mtrue[h];
      mx = fmaxf(mx, xor8(mx));
      mx = max_lane_groups(mx);
      mref[h] = uniform_f(mx);
    }
    fixed_ref = true;
  }

  // merge the token groups (lanes with equal lane % LPT): each lane's state
  // with its partner's at distance 8 (DPP), 16 and 32 (permlane swaps), all
  // in VALU.  Every lane's weights are relative to the same wave-uniform
  // reference max, so merging two lanes' states is a plain sum.
  auto merge_step = [&](auto off_tag) {
    constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float l0, l1, t0, t1;
      lane_pair<OFF>(l[h], l0, l1);
      lane_pair<OFF>(mtrue[h], t0, t1);
      l[h] = l0 + l1;
      if constexpr (BF16) {
        float r0, r1;
        lane_pair<OFF>(lr[h], r0, r1);
        lr[h] = r0 + r1;
      }
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        float o0, o1;
        lane_pair<OFF>(o[h][e], o0, o1);
        o[h][e] = o0 + o1;
      }
      mtrue[h] = fmaxf(t0, t1);
    }
  };
  if constexpr (LPT == 8) merge_step(std::integral_constant<int, 8>{});
  merge_step(std::integral_constant<int, 16>{});
  merge_step(std::integral_constant<int, 32>{});

  // lanes 0..LPT-1 hold the result: O normalised (by the weights P.V used), m (true max), the
  // exact l relative to it
  float inv[R], lt[R];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    inv[h] = 1.f / (BF16 ? lr[h] : l[h]);
    lt[h] = l[h] * fast_exp2(mref[h] - mtrue[h]);
  }
  const bool last_by_count = E > 1 && __builtin_amdgcn_readfirstlane(cval) == E - 1;
  if (E == 1 || last_by_count) {
    if (E == 1) {
      if (ts == 0) {
#pragma unroll
        for (int h = 0; h < R; ++h) {
          const int64_t row = (int64_t)qi * p.hq + kvh * R + h;
#pragma unroll
          for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int q4 = 0; q4 < EPC / 4; ++q4) {
              const int e = k * EPC + q4 * 4;
              f32x4 v = {o[h][e] * inv[h], o[h][e + 1] * inv[h], o[h][e + 2] * inv[h], o[h][e + 3] * inv[h]};
              store_out4(p, row * D + (k * LPT + c) * EPC + q4 * 4, v);
            }
          if (c == 0) store_ml(p, row, mtrue[h], lt[h]);
        }
      }
    } else {
      // every other piece had arrived: the merge of the E partials in slot
      // order, this wave's own (slot jown) from its registers through LDS,
      // so that all 64 lanes load the other pieces at once
      __attribute__((address_space(3))) float* own =
          (__attribute__((address_space(3))) float*)(smem + S::OWN_BASE + wave * S::OWN_STRIDE);
      if (ts == 0) {
#pragma unroll
        for (int h = 0; h < R; ++h)
#pragma unroll
          for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int q4 = 0; q4 < EPC / 4; ++q4) {
              const int e = k * EPC + q4 * 4;
              *(__attribute__((address_space(3))) f32x4*)(own + h * D + (k * LPT + c) * EPC + q4 * 4) =
                  f32x4{o[h][e] * inv[h], o[h][e + 1] * inv[h], o[h][e + 2] * inv[h], o[h][e + 3] * inv[h]};
            }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      merge_pieces<D, R>(p, qi, kvh, E, slot / p.hkv - (int)p.slot_off[qi], own, mtrue, lt);
    }
    if (E > 1 && lane == 0) reset_counter(ctr);  // no other piece touches it in this launch
    return;
  }
  // a partial, then the arrival; the last arriver merges
  if (ts == 0) {
    const auto ro = make_rsrc(p.part_o, p.part_o_bytes);
    const auto rm = make_rsrc(p.part_ml, p.part_ml_bytes);
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const uint32_t srow = (uint32_t)(slot * R + h);
#pragma unroll
      for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int q4 = 0; q4 < EPC / 4; ++q4) {
          const int e = k * EPC + q4 * 4;
          f32x4 v = {o[h][e] * inv[h], o[h][e + 1] * inv[h], o[h][e + 2] * inv[h], o[h][e + 3] * inv[h]};
          st_coh4(ro, (srow * D + (k * LPT + c) * EPC + q4 * 4) * 4u, v);
        }
      if (c == 0) {
        st_coh1(rm, srow * 8u, mtrue[h]);
        st_coh1(rm, srow * 8u + 4u, lt[h]);
      }
    }
  }
  release_partials();
  int old = 0;
  if (lane == 0) old = arrive_counter(ctr);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old == E - 1) {
    merge_wave<D, R>(p, qi, kvh);
    if (lane == 0) reset_counter(ctr);
  }
}

// ------------------------------------------------------- MFMA prefix tile ---
// Rows = (member query, head in kv group) pairs of one group, up to 128 rows
// in 16-row slices (2 per wave), against one prefix chunk staged through LDS
// 64 tokens (4 pages) at a time.  K and V are copied global -> LDS by the
// load unit (global_load_lds_dwordx4, no registers), double buffered in two
// separate LDS arrays: block b+1 is in flight while block b is computed.
// Wave w copies page w of every 64-token block.
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16: A = K rows (tokens), B = Q^T.
//   O^T = V^T P^T with the same MFMA: A = V^T read from the row-major V tile
//   with ds_read_b64_tr_b16 (transposing 4x16 bf16 blocks on the way), B = P^T.
// K rows feed the 16-row MFMA in the order token = 8*(m/4) + 4*half + m%4
// (half = which 16-token tile of a 32-token block), so the S^T accumulator
// of lane group g holds 8 consecutive tokens, exactly the k-slice lane group
// g supplies as the B operand (P^T) of the PV product: P stays in registers.
// Rows of K and V are stored with their 16-byte chunks XOR-swizzled by a key
// of the token that makes both the K operand reads (16 tokens, one chunk)
// and the transposing V reads (4 tokens x 32 bytes per lane group) hit
// distinct LDS banks.
template <int D>
struct MfShape {
  static constexpr int KK = D / 32;            // k-steps of the QK product
  static constexpr int NB = D / 16;            // 16-wide dim blocks of O
  static constexpr int TILE = MfLayout<D>::TILE;
  static constexpr int NI = MfLayout<D>::NI;   // 1 KiB copies per wave per tile
  static constexpr int STAGE = 2 * TILE;       // K then V
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 layout: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// A wave-uniform 64-bit address in scalar registers, whatever the register
// allocator did with the arithmetic that made it (readfirstlane yields a
// signed int: each half is widened as unsigned).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t a) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// Copy 16 bytes per lane from kbase + voff to LDS at lds_k + 16 * lane and
// from vbase + voff to lds_v + 16 * lane, through the load unit
// (global_load_lds_dwordx4, saddr form; M0 holds the LDS destination and is
// restored: the compiler reserves it).  Written as inline asm so that the
// compiler does not make every later LDS read wait for these copies:
// completion is awaited explicitly with s_waitcnt vmcnt, followed by a
// barrier.  The "memory" clobber tells the compiler that LDS may change.
__device__ __forceinline__ void copy_kv_to_lds(uint64_t kbase, uint64_t vbase, uint32_t voff, uint32_t lds_k,
                                               uint32_t lds_v) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %4\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_k), "s"(lds_v), "v"(voff), "s"(kbase), "s"(vbase)
      : "memory");
}

// Workgroup barrier ordering LDS accesses only (no wait for global memory,
// so copies into the other stage stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// Running state of a wave's NS row slices.
template <int D>
struct MfRows {
  bf16x8 qb[2][D / 32];        // Q^T B operands
  f32x4 o[2][D / 16];          // O^T accumulators (unnormalised, relative to mref)
  f32x4 rsum[2];               // row sums of the bf16-rounded weights (every element)
  float mref[2];               // reference max of the row (lazy), log2 units
  float mtrue[2];              // max of the row's scores this lane has seen, log2 units
  float lrow[2];               // this lane's part of the row sum of exact weights
  int koff[D / 32];            // this lane's LDS offsets of the tile-0 K operand reads
  int voff[D / 16];            // and of the (kb 0, hf 0) V^T operand reads
};

// One 64-token block (K at Ks, V at Vs) for the wave's NS slices; tokens at or
// past `valid` are masked, and with `limits` set, tokens at or past the
// lane's row limit limb[sl] (both counted from the block's first token).
template <int D, int NS, typename Copy>
__device__ __forceinline__ void mf_block(MfRows<D>& st, const lds_char* Ks, const lds_char* Vs, int valid, float sc,
                                         const bf16x8& ones, bool limits, const int (&limb)[2], Copy&& copy) {
  constexpr int KK = D / 32, NB = D / 16;
  const int lg = (threadIdx.x & 63) >> 4;
  // ---- S^T tiles: t = kb*2 + half covers tokens 32kb + {8*(m/4) + 4*half + m%4} ----
  f32x4 s[NS][4];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl)
#pragma unroll
    for (int t = 0; t < 4; ++t) s[sl][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The QK product by k-step: the MFMAs of one k-step over the four token
  // tiles and NS slices are 4 NS independent accumulation chains (a single
  // wave issues back-to-back MFMAs at full rate only with about eight in
  // flight; a chain's next MFMA waits for the previous result).  The K
  // operands of k-steps kk and kk + 1 are in flight while kk - 1's MFMAs
  // issue; pieces of the next block's copy follow each k-step's MFMAs, so
  // that a stall on issuing one (the load path is shared with the other
  // workgroup on the CU) leaves queued matrix work behind it.
  bf16x8 a[2][4];
  auto kread = [&](int kk) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      a[kk & 1][t] = *(const __attribute__((address_space(3))) bf16x8*)(Ks + st.koff[kk] + mf_k_step<D>(t));
  };
  kread(0);
  if (KK > 1) kread(1);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int sl = 0; sl < NS; ++sl)
        s[sl][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk & 1][t], st.qb[sl][kk], s[sl][t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (kk + 2 < KK) kread(kk + 2);
#pragma unroll
    for (int c = kk * 4 / KK; c < (kk + 1) * 4 / KK; ++c) copy(c);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (valid < 64 || limits) {  // last block of the chunk, or rows with their own limits
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const int lim = min(valid, limb[sl]) - 8 * lg;  // against the token's offset from 8 lg
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((t >> 1) * 32 + 4 * (t & 1) + i >= lim) s[sl][t][i] = -INFINITY;
    }
  }
  // ---- online softmax per row (lane's row = l16; 16 raw scores per lane) ----
  // Each lane checks its own scores against the row's reference max; only
  // when one exceeds it by kLazy (rare) does the wave take the row maxima
  // across lane groups and rescale.  Maxima and the rescale come first, so
  // that the exponentials and the P.V products after them form one
  // branch-free stretch.
  float mx[NS];
  bool up = false;
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, s[sl][t][i]);
    mx[sl] = m * sc;  // log2 units (sc > 0 keeps the order)
    st.mtrue[sl] = fmaxf(st.mtrue[sl], mx[sl]);
    up |= mx[sl] > st.mref[sl] + kLazy;
  }
  if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const float mn = fmaxf(st.mref[sl], max_lane_groups(mx[sl]));
      const float alpha = fast_exp2(st.mref[sl] - mn);  // 1 for a slice that did not move
      st.mref[sl] = mn;
      st.lrow[sl] *= alpha;
      st.rsum[sl] *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) st.o[sl][nb] *= alpha;
    }
  }
  // ---- P (bf16) and O^T += V^T P^T by 32-token k-slice kb; V^T through
  // transposing LDS reads.  The k-slice-1 weights are computed in pieces
  // between the k-slice-0 MFMAs (the scheduler is fenced per step), so the
  // exponentials overlap the matrix core; V^T operands are read one step
  // ahead. ----
  bf16x8 pb[NS][2];
  float ps[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) ps[sl] = 0.f;
  // two weights of slice sl, k-slice kb: token tile t = 2 kb + (piece >> 1),
  // accumulator elements 2 (piece & 1) and 2 (piece & 1) + 1
  auto wpiece = [&](int sl, int kb, int piece) {
    const int t = kb * 2 + (piece >> 1), i0 = 2 * (piece & 1);
    const float nm = -st.mref[sl];
    const float p0 = fast_exp2(fmaf(s[sl][t][i0], sc, nm));  // exp2(-inf) = 0 when masked
    const float p1 = fast_exp2(fmaf(s[sl][t][i0 + 1], sc, nm));
    ps[sl] += p0 + p1;
    const int e = (piece >> 1) * 4 + i0;
    pb[sl][kb][e] = (__bf16)p0;
    pb[sl][kb][e + 1] = (__bf16)p1;
  };
  // row sum of the bf16-rounded weights used in P.V, by MFMA against ones
  auto rowsum = [&](int kb) {
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
      st.rsum[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[sl][kb], st.rsum[sl], 0, 0, 0);
  };
  auto vread = [&](int kb, int nb) {
    v4i16 h[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      h[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(Vs + st.voff[nb] + mf_v_step<D>(kb, hf)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
#pragma unroll
  for (int sl = 0; sl < NS; ++sl)
#pragma unroll
    for (int piece = 0; piece < 4; ++piece) wpiece(sl, 0, piece);
  rowsum(0);
  bf16x8 vn = vread(0, 0);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bf16x8 va = vn;
    vn = nb + 1 < NB ? vread(0, nb + 1) : vread(1, 0);
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) st.o[sl][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[sl][0], st.o[sl][nb], 0, 0, 0);
    if (nb < NS * 4) wpiece(nb / 4, 1, nb % 4);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = NB; q < NS * 4; ++q) wpiece(q / 4, 1, q % 4);  // (D 64: fewer steps than pieces)
  rowsum(1);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bf16x8 va = vn;
    if (nb + 1 < NB) vn = vread(1, nb + 1);
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) st.o[sl][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[sl][1], st.o[sl][nb], 0, 0, 0);
  }
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) st.lrow[sl] += ps[sl];
}

template <int D, int R>
__device__ __forceinline__ void prefix_mfma_tile(const DecodeParams& p, const WorkItem& it, lds_char* stage0, lds_char* stage1) {
  using S = MfShape<D>;
  constexpr int KK = S::KK, NB = S::NB, NI = S::NI;
  constexpr int ROW = MfLayout<D>::ROW, TILEB = 16 * D * 2;  // bytes of one (page, kv head) tile
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int kvh = it.kvh, rb = it.a, rc = it.b, jslot = it.kind >> 8;
  const int ntok = it.tok_end - it.tok_begin, npages = (ntok + 15) >> 4, nblocks = (ntok + 63) >> 6;
  const int nslices = (rc + 15) >> 4;
  const int ns = wave + kWaves < nslices ? 2 : (wave < nslices ? 1 : 0);
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  const char* kp = reinterpret_cast<const char*>(p.k);
  const char* vp = reinterpret_cast<const char*>(p.v);

  // The loads before the loop form two short chains that run side by side:
  // page ids -> copy of block 0, and member queries -> Q rows.  (Rows are
  // counted over the whole member array, so no group offset is read first.)
  // Lane j holds the id of the page this wave copies in block j (page 4j+wave
  // of the chunk, clamped to its last page); a chunk has at most 32 blocks.
  int pid_v = 0;
  if (lane < nblocks) pid_v = p.pages[it.page_base + min(lane * 4 + wave, npages - 1)];
  int qrow[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int row = (wave + kWaves * sl) * 16 + l16;
    qrow[sl] = (sl < ns && row < rc) ? p.members[(rb + row) / R] : -1;
  }
  // Prefix tokens of this chunk the lane's row sees (a query with a prefix
  // limit, e.g. a prefill token, sees keys before its own position only);
  // lmin = the wave's smallest, to find the blocks that need the masks.
  int lim[2] = {kNoLimit, kNoLimit};
  int lmin = kNoLimit;
  if (p.qlim) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
      if (qrow[sl] >= 0) lim[sl] = p.qlim[qrow[sl]] - it.tok_begin;
    int v = min(lim[0], lim[1]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = min(v, __shfl_xor(v, o));
    lmin = __builtin_amdgcn_readfirstlane(v);
  }

  // copy of one 64-token block into a stage, global -> LDS through the load
  // unit: this wave's NI loads per tile (index maps in layout.h) all fall in
  // one page.  Tokens past the chunk re-read its last token so every LDS row
  // stays finite (their scores are masked).
  int tin[NI], coff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    tin[i] = mf_copy_token<D>(wave, i, lane) & 15;
    coff[i] = mf_copy_chunk<D>(wave, i, lane) * 16;
  }
  const int64_t tile_stride = (int64_t)p.hkv * TILEB;
  // where this wave's copy of block blk comes from: K and V tile bases and
  // the token clamp (tokens past the chunk re-read its last token)
  // (scalar bases, computed once per block; clamp is false unless this
  // wave's page reaches past the chunk)
  struct Src {
    uint64_t ks, vs;
    int du, lim;
    bool clamp;
  };
  auto src = [&](int blk) {
    const int pg = min(blk * 4 + wave, npages - 1);
    const int pid = __builtin_amdgcn_readlane(pid_v, blk);
    const int64_t tile = (int64_t)pid * tile_stride + (int64_t)kvh * TILEB;
    // du > 0 only when this wave's page is past the chunk; lim = last valid token within the page
    const int du = (blk * 4 + wave - pg) * 16, lim = ntok - 1 - pg * 16;
    return Src{uniform_u64(reinterpret_cast<uint64_t>(kp + tile)), uniform_u64(reinterpret_cast<uint64_t>(vp + tile)),
               du, lim, du > 0 || lim < 15};
  };
  // this lane's source offset of load i in an unclamped page
  uint32_t off0[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) off0[i] = (uint32_t)(tin[i] * ROW + coff[i]);
  // load i (of NI) of K and of V into a stage; lane l lands at +16 l
  // (a branch on the uniform clamp flag, not a select: the common path
  // issues no offset arithmetic)
  auto dma_piece = [&](const Src& c, lds_char* stage, int i) {
    const uint32_t dst = (uint32_t)(uintptr_t)stage + (uint32_t)((wave * NI + i) * 1024);
    if (__builtin_expect(c.clamp, 0)) {
      const uint32_t off = (uint32_t)(min(tin[i] + c.du, c.lim) * ROW + coff[i]);
      copy_kv_to_lds(c.ks, c.vs, off, dst, dst + S::TILE);
    } else {
      copy_kv_to_lds(c.ks, c.vs, off0[i], dst, dst + S::TILE);
    }
  };
  {
    const Src c = src(0);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma_piece(c, stage0, i);
  }

  MfRows<D> st;
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qrow[sl] >= 0) {
        const int grow = rb + (wave + kWaves * sl) * 16 + l16;
        const int64_t off = ((int64_t)qrow[sl] * p.hq + kvh * R + grow % R) * D + kk * 32 + lg * 8;
        w = *reinterpret_cast<const u32x4*>(qp + off);
      }
      st.qb[sl][kk] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st.o[sl][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.rsum[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.mref[sl] = kNoMax;
    st.mtrue[sl] = -INFINITY;
    st.lrow[sl] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) st.koff[kk] = mf_k_base<D>(kk, lg, l16);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.voff[nb] = mf_v_base<D>(nb, lg, l16);
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  const float sc = p.scale_log2;
  // Use the loaded registers once here, so that the compiler waits for their
  // loads before the block loop rather than at a first use inside it (a wait
  // there would also wait for the copies in flight).
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(st.qb[sl][kk]));
  asm volatile("" ::"v"(pid_v));
  // the LDS offsets are held in registers for the whole loop
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(st.koff[kk]));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(st.voff[nb]));

  // Arrival counters of the rows' (query, kv head) pairs, read by the head-0
  // lane of each query when the last block starts: if every other piece has
  // arrived by then, the tile merges in registers at the end.  (A piece that
  // arrives later is merged the slow way: read or written, the decision is
  // sound.)
  int cval[2] = {-1, -1};
  auto read_counters = [&]() {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int grow = rb + (wave + kWaves * sl) * 16 + l16;
      if (qrow[sl] >= 0 && lim[sl] > 0 && lg == 0 && grow % R == 0 && p.expected[qrow[sl]] > 1)
        cval[sl] = __hip_atomic_load(p.counters + (int64_t)qrow[sl] * p.hkv + kvh, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // even blocks in stage0, odd blocks in stage1; the copy of block b+1 is
  // issued before block b is computed.  The loop is instantiated per slice
  // count, so a wave's state never crosses a branch inside it.
  auto run = [&](auto ns_tag) {
    constexpr int NSL = decltype(ns_tag)::value;
    // compute block blk from `stage` while copying block blk + 1 (if any) into `next`
    auto compute = [&](const lds_char* stage, int blk, lds_char* next) {
      const bool more = blk + 1 < nblocks;
      const Src c = src(more ? blk + 1 : blk);
      auto copy = [&](int t) {  // NI pieces spread over the 4 token tiles
        if (more) {
#pragma unroll
          for (int i = t * NI / 4; i < (t + 1) * NI / 4; ++i) dma_piece(c, next, i);
        }
      };
      if constexpr (NSL > 0) {
        const int limb[2] = {lim[0] - blk * 64, lim[1] - blk * 64};
        mf_block<D, NSL>(st, stage, stage + S::TILE, min(64, ntok - blk * 64), sc, ones, lmin < blk * 64 + 64, limb,
                         copy);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) copy(t);
      }
    };
    // one barrier per block: after it every wave's copy of block b has landed
    // and every wave is done with block b - 1, whose stage then receives the
    // copy of block b + 1 (issued in pieces while block b is computed)
    for (int blk = 0; blk < nblocks; blk += 2) {
      __builtin_amdgcn_s_waitcnt(wait_vm(0));  // this wave's copy of block blk
      lds_barrier();
      if (blk + 1 == nblocks) read_counters();
      compute(stage0, blk, stage1);
      if (blk + 1 >= nblocks) break;
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      lds_barrier();
      if (blk + 2 == nblocks) read_counters();
      compute(stage1, blk + 1, stage0);
    }
  };
  if (ns == 2)
    run(std::integral_constant<int, 2>{});
  else if (ns == 1)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});

  // ---- per row: the output (the chunk is the whole context), a merge in
  // registers (every other piece of the (query, kv head) had arrived when the
  // last block started), or a partial and an arrival.  Both slices' memory
  // operations are issued together, so the epilogue costs few round trips.
  const auto ro = make_rsrc(p.part_o, p.part_o_bytes);
  const auto rm = make_rsrc(p.part_ml, p.part_ml_bytes);
  bool valid[2], head[2];
  int qi[2], hh[2], E[2], dec[2];
  float inv[2], mt[2], lt[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    valid[sl] = head[sl] = false;
    qi[sl] = hh[sl] = dec[sl] = 0;
    E[sl] = 1;
    inv[sl] = mt[sl] = lt[sl] = 0.f;
    if (sl >= ns) continue;  // wave-uniform
    float L = st.lrow[sl], L0, L1;
    lane_pair<32>(L, L0, L1);
    L = L0 + L1;
    lane_pair<16>(L, L0, L1);
    L = L0 + L1;
    const float Lr = st.rsum[sl][0];  // every element holds the row's sum
    mt[sl] = max_lane_groups(st.mtrue[sl]);
    const int row = (wave + kWaves * sl) * 16 + l16;
    valid[sl] = row < rc && lim[sl] > 0;  // (a row whose limit ends before the chunk has no piece here)
    hh[sl] = (rb + row) % R;  // a query's R rows lie in one slice (R divides 16)
    qi[sl] = valid[sl] ? qrow[sl] : 0;
    inv[sl] = 1.f / Lr;  // normalise with the sum of the rounded weights used in P.V
    lt[sl] = L * fast_exp2(st.mref[sl] - mt[sl]);
    E[sl] = valid[sl] ? p.expected[qi[sl]] : 1;
    // the head-0 lane of each query has read the arrival counter: 1 = every
    // other piece had arrived (merge here), 2 = write a partial and arrive
    head[sl] = valid[sl] && lg == 0 && hh[sl] == 0;
    int d = 0;
    if (head[sl] && E[sl] > 1) d = cval[sl] == E[sl] - 1 ? 1 : 2;
    dec[sl] = __shfl(d, l16 - hh[sl]);  // the query's head-0 row, lane group 0
  }
  // Partials first: their stores must be complete before the arrival, and
  // the arrivals' round trip then overlaps the loads of the merges below.
  bool wrote = false;
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (!(valid[sl] && E[sl] > 1 && dec[sl] == 2)) continue;
    wrote = true;
    const uint32_t srow = (uint32_t)(((p.slot_off[qi[sl]] + jslot) * p.hkv + kvh) * R + hh[sl]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st_coh4(ro, (srow * D + nb * 16 + lg * 4) * 4u, st.o[sl][nb] * inv[sl]);
    if (lg == 0) {
      st_coh1(rm, srow * 8u, mt[sl]);
      st_coh1(rm, srow * 8u + 4u, lt[sl]);
    }
  }
  const bool any_partial = __builtin_amdgcn_ballot_w64(wrote) != 0;
  if (any_partial) release_partials();
  // arrivals (one wave holds all rows of a query); counters of pairs merged
  // here go back to zero (no other piece touches them in this launch)
  int old[2] = {0, 0};
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    int32_t* ctr = p.counters + (int64_t)qi[sl] * p.hkv + kvh;
    if (head[sl] && dec[sl] == 1) reset_counter(ctr);
    if (head[sl] && dec[sl] == 2) old[sl] = arrive_counter(ctr);
  }
  // the other piece of two-piece merges, both slices at once
  f32x4 oo[2][NB];
  float mo[2] = {0.f, 0.f}, lo[2] = {0.f, 0.f};
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (!(valid[sl] && E[sl] == 2 && dec[sl] == 1)) continue;
    const uint32_t srow = (uint32_t)(((p.slot_off[qi[sl]] + (1 - jslot)) * p.hkv + kvh) * R + hh[sl]);
    mo[sl] = ld_coh1(rm, srow * 8u);
    lo[sl] = ld_coh1(rm, srow * 8u + 4u);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oo[sl][nb] = ld_coh4(ro, (srow * D + nb * 16 + lg * 4) * 4u);
  }
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (!valid[sl]) continue;
    const int64_t orow = (int64_t)qi[sl] * p.hq + kvh * R + hh[sl];
    if (E[sl] == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) store_out4(p, orow * D + nb * 16 + lg * 4, st.o[sl][nb] * inv[sl]);
      if (lg == 0) store_ml(p, orow, mt[sl], lt[sl]);
    } else if (dec[sl] == 1) {
      // the merge of the E partials in slot order, with the operations of
      // merge_wave (uncontracted), this tile's own partial (slot jslot) taken
      // from registers
#pragma clang fp contract(off)
      if (E[sl] == 2) {
        const float m0 = jslot == 0 ? mt[sl] : mo[sl], m1 = jslot == 0 ? mo[sl] : mt[sl];
        const float l0 = jslot == 0 ? lt[sl] : lo[sl], l1 = jslot == 0 ? lo[sl] : lt[sl];
        const float M = fmaxf(fmaxf(kNoMax, m0), m1);
        const float w0 = l0 * fast_exp2(m0 - M), w1 = l1 * fast_exp2(m1 - M);
        float Ls = 0.f;
        Ls += w0;
        Ls += w1;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const f32x4 own = st.o[sl][nb] * inv[sl];
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
          acc += w0 * (jslot == 0 ? own : oo[sl][nb]);
          acc += w1 * (jslot == 0 ? oo[sl][nb] : own);
          store_out4(p, orow * D + nb * 16 + lg * 4, acc * (1.f / Ls));
        }
        if (lg == 0) store_ml(p, orow, M, Ls);
      } else if (E[sl] > kMergeUnroll) {
        const int64_t s0 = p.slot_off[qi[sl]];
        float M = kNoMax;
        for (int j = 0; j < E[sl]; ++j) {
          const uint32_t srow = (uint32_t)(((s0 + j) * p.hkv + kvh) * R + hh[sl]);
          M = fmaxf(M, j == jslot ? mt[sl] : ld_coh1(rm, srow * 8u));
        }
        float Ls = 0.f;
        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < E[sl]; ++j) {
          const uint32_t srow = (uint32_t)(((s0 + j) * p.hkv + kvh) * R + hh[sl]);
          if (j == jslot) {
            const float w = lt[sl] * fast_exp2(mt[sl] - M);
            Ls += w;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] += w * (st.o[sl][nb] * inv[sl]);
          } else {
            const float w = ld_coh1(rm, srow * 8u + 4u) * fast_exp2(ld_coh1(rm, srow * 8u) - M);
            Ls += w;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] += w * ld_coh4(ro, (srow * D + nb * 16 + lg * 4) * 4u);
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) store_out4(p, orow * D + nb * 16 + lg * 4, acc[nb] * (1.f / Ls));
        if (lg == 0) store_ml(p, orow, M, Ls);
      }
    }
  }
  // three-piece merges, after the two-piece ones (whose loads are dead by then)
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (!(valid[sl] && E[sl] == 3 && dec[sl] == 1)) continue;
    const int64_t orow = (int64_t)qi[sl] * p.hq + kvh * R + hh[sl];
    {
#pragma clang fp contract(off)
      // the two other pieces' m, l and O rows, all loads in flight together
      // (one slice at a time: the scheduler is fenced around it)
      __builtin_amdgcn_sched_barrier(0);
      const int64_t s0 = p.slot_off[qi[sl]];
      const int ja = jslot == 0 ? 1 : 0, jb = jslot == 2 ? 1 : 2;  // the other slots, in order
      float mo2[2], lo2[2];
      f32x4 oo2[2][NB];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint32_t srow = (uint32_t)(((s0 + (x ? jb : ja)) * p.hkv + kvh) * R + hh[sl]);
        mo2[x] = ld_coh1(rm, srow * 8u);
        lo2[x] = ld_coh1(rm, srow * 8u + 4u);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oo2[x][nb] = ld_coh4(ro, (srow * D + nb * 16 + lg * 4) * 4u);
      }
      // slot j's piece: this tile's own, or the x-th other
      auto xof = [&](int j) { return j == ja ? 0 : 1; };
      float M = kNoMax;
#pragma unroll
      for (int j = 0; j < 3; ++j) M = fmaxf(M, j == jslot ? mt[sl] : mo2[xof(j)]);
      float w[3], Ls = 0.f;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        w[j] = j == jslot ? lt[sl] * fast_exp2(mt[sl] - M) : lo2[xof(j)] * fast_exp2(mo2[xof(j)] - M);
        Ls += w[j];
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4 own = st.o[sl][nb] * inv[sl];
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 3; ++j) acc += w[j] * (j == jslot ? own : oo2[xof(j)][nb]);
        store_out4(p, orow * D + nb * 16 + lg * 4, acc * (1.f / Ls));
      }
      if (lg == 0) store_ml(p, orow, M, Ls);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // merges of four or more pieces, last (one slice at a time)
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (!(valid[sl] && E[sl] > 3 && E[sl] <= kMergeUnroll && dec[sl] == 1)) continue;
    const int64_t orow = (int64_t)qi[sl] * p.hq + kvh * R + hh[sl];
    __builtin_amdgcn_sched_barrier(0);
    {
#pragma clang fp contract(off)
      // m and l of every piece in one batch of loads, then the O rows piece
      // by piece (slot order throughout)
      const int64_t s0 = p.slot_off[qi[sl]];
      const int En = E[sl];
      auto srow_of = [&](int j) { return (uint32_t)(((s0 + j) * p.hkv + kvh) * R + hh[sl]); };
      float mj[kMergeUnroll], lj[kMergeUnroll];
#pragma unroll
      for (int j = 0; j < kMergeUnroll; ++j) {
        mj[j] = mt[sl];
        lj[j] = lt[sl];
        if (j < En && j != jslot) {
          mj[j] = ld_coh1(rm, srow_of(j) * 8u);
          lj[j] = ld_coh1(rm, srow_of(j) * 8u + 4u);
        }
      }
      float M = kNoMax;
#pragma unroll
      for (int j = 0; j < kMergeUnroll; ++j)
        if (j < En) M = fmaxf(M, mj[j]);
      float Ls = 0.f;
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMergeUnroll; ++j) {
        if (j >= En) break;
        const float w = lj[j] * fast_exp2(mj[j] - M);
        Ls += w;
        if (j == jslot) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[nb] += w * (st.o[sl][nb] * inv[sl]);
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[nb] += w * ld_coh4(ro, (srow_of(j) * D + nb * 16 + lg * 4) * 4u);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) store_out4(p, orow * D + nb * 16 + lg * 4, acc[nb] * (1.f / Ls));
      if (lg == 0) store_ml(p, orow, M, Ls);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last arrivers among the partials written above merge
  if (any_partial) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      uint64_t lm = __builtin_amdgcn_ballot_w64(head[sl] && dec[sl] == 2 && old[sl] == E[sl] - 1);
      while (lm) {
        const int src = __builtin_ctzll(lm);
        lm &= lm - 1;
        const int q = __builtin_amdgcn_readlane(qi[sl], src);
        merge_wave<D, R>(p, q, kvh);
        if (lane == 0) reset_counter(p.counters + (int64_t)q * p.hkv + kvh);
      }
    }
  }
}

// Empty partial (0, -inf, 0) of every head of a query the plan does not
// cover (PREFIX_ONLY / DISTINCT_ONLY plans); one wave.
template <int D>
__device__ __forceinline__ void empty_wave(const DecodeParams& p, const WorkItem& it) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)it.id * p.hq;
  for (int el = lane * 4; el < p.hq * D; el += 256) store_out4(p, base * D + el, f32x4{0.f, 0.f, 0.f, 0.f});
  for (int h = lane; h < p.hq; h += 64) {
    if (p.out_m) p.out_m[base + h] = -INFINITY;
    if (p.out_l) p.out_l[base + h] = 0.f;
  }
}

// The workspace does not hold the launching plan's image (overwritten since
// its upload): every output element becomes NaN, so the failure is loud, and
// nothing else is read from the workspace.  Grid-stride over the outputs.
template <int D>
__device__ __forceinline__ void poison_outputs(const DecodeParams& p) {
  const int64_t rows = (int64_t)p.num_queries * p.hq;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows * D; i += stride) {
    if (p.out_bf16)
      reinterpret_cast<uint16_t*>(p.out)[i] = 0x7fc0u;
    else
      reinterpret_cast<float*>(p.out)[i] = __builtin_nanf("");
    if (i < rows) {
      if (p.out_m) p.out_m[i] = __builtin_nanf("");
      if (p.out_l) p.out_l[i] = __builtin_nanf("");
    }
  }
}

// LDS: two stages of the MFMA tile (the first also holds the mat-vec tiles'
// q rows) and the tile's arrival list; separate arrays, so the compiler can
// tell a stage's reads from the copy into the other stage.
template <int D, int R, bool BF16>
struct Lds {
  static constexpr int MV = MvShape<D, R, BF16>::LDS_BYTES;
  static_assert(kWaves == 4, "the mat-vec LDS layout assumes four waves");
  static constexpr int MF = BF16 ? MfShape<D>::STAGE : 16;
  static constexpr int STAGE0 = MV > MF ? MV : MF;
};

template <int D, int R, bool BF16>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds0[Lds<D, R, BF16>::STAGE0];
  __shared__ __attribute__((aligned(16))) char lds1[Lds<D, R, BF16>::MF];
  const uint64_t t0 = p.trace ? __builtin_amdgcn_s_memrealtime() : 0;
  const WorkItem* unit = p.items + (int64_t)blockIdx.x * kUnitItems;
  // The image header, the unit's first word and this wave's item load
  // together (one wait): a mat-vec wave then starts its page table and q
  // loads one round trip earlier.  (The unit lies inside the image the host
  // checked; nothing loaded is used before the header is.)
  const uint64_t hdr = *reinterpret_cast<const uint64_t*>(p.header);
  const int word0 = unit[0].kind;
  const WorkItem it = unit[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
  asm volatile("" ::"s"(hdr), "s"(word0), "s"(it.kind), "s"(it.tok_end), "s"(it.b));
  if (hdr != (((uint64_t)p.plan_id << 32) | kImageMagic)) {
    poison_outputs<D>(p);
    return;
  }
  const int kind0 = word0 & 0xff;
  if (kind0 == ITEM_PREFIX_MFMA) {
    if constexpr (BF16)
      prefix_mfma_tile<D, R>(p, unit[0], (lds_char*)lds0, (lds_char*)lds1);
  } else {
    const int kind = it.kind & 0xff;
    if (kind == ITEM_MATVEC)
      matvec_wave<D, R, BF16>(p, it, lds0);
    else if (kind == ITEM_EMPTY)
      empty_wave<D>(p, it);
  }
  if (p.trace) {  // per-unit timing: start, end of the whole workgroup, where it ran
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
      const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID
      const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20);  // XCC_ID
      uint64_t* t = p.trace + (int64_t)blockIdx.x * 4;
      t[0] = t0;
      t[1] = t1;
      t[2] = hw | ((uint64_t)xcc << 32);
      t[3] = (uint64_t)kind0;
    }
  }
}

template <int D, int R, bool BF16>
static hipError_t launch(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<D, R, BF16>), dim3(p.num_units), dim3(kThreads), 0, s, p);
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
  if (p.num_units <= 0) return hipSuccess;
  if (head_dim == 64) return bf16 ? launch_r<64, true>(p, r, s) : launch_r<64, false>(p, r, s);
  if (head_dim == 128) return bf16 ? launch_r<128, true>(p, r, s) : launch_r<128, false>(p, r, s);
  return hipErrorInvalidValue;
}

}  // namespace psa
