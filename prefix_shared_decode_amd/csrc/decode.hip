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

#include "layout.h"
#include "psa_internal.h"

namespace psa {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNoMax = -1.0e30f;  // reference max of an empty state (finite: exp2 stays NaN-free)
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
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kSc1 = 16;  // cache policy: coherent at device (agent) scope

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
// output; one wave.  Partials hold O normalised, m (log2 units), l.
template <int D, int R>
__device__ void merge_wave(const DecodeParams& p, int qi, int kvh) {
  const int lane = threadIdx.x & 63;
  const int E = p.expected[qi];
  const int64_t s0 = p.slot_off[qi];
  const auto ro = make_rsrc(p.part_o, p.part_o_bytes);
  const auto rm = make_rsrc(p.part_ml, p.part_ml_bytes);
  constexpr int C4 = D / 4;  // float4 chunks per row
  for (int ci = lane; ci < R * C4; ci += 64) {
    const int hh = ci / C4, c4 = ci % C4;
    float M = kNoMax;
    for (int j = 0; j < E; ++j) {
      const uint32_t slot = (uint32_t)(((s0 + j) * p.hkv + kvh) * R + hh);
      M = fmaxf(M, ld_coh1(rm, slot * 8u));
    }
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < E; ++j) {
      const uint32_t slot = (uint32_t)(((s0 + j) * p.hkv + kvh) * R + hh);
      const float w = ld_coh1(rm, slot * 8u + 4u) * fast_exp2(ld_coh1(rm, slot * 8u) - M);
      L += w;
      acc += w * ld_coh4(ro, (slot * D + c4 * 4) * 4u);
    }
    const int64_t row = (int64_t)qi * p.hq + kvh * R + hh;
    store_out4(p, row * D + c4 * 4, acc * (1.f / L));
    if (c4 == 0) store_ml(p, row, M, L);
  }
}

// ----------------------------------------------------------- mat-vec tile ---
// One wave, one (query, kv head, token chunk).  LPT consecutive lanes hold one
// token: lane c = lane % LPT covers the 16-byte chunks k*LPT + c of the
// token's row (k < NCH), so each load instruction reads 64/LPT whole tokens as
// contiguous runs; a page (16 tokens) is NT = LPT/4 token slots per lane.  All
// R query heads of the kv head share one read of the page.  Scores are summed
// over the LPT lanes with DPP; P.V uses bf16 dot2 over pairs of the lane's
// tokens.  LPT is 8 unless R * dims-per-lane would exceed 64 accumulators.
// The next page is in flight while one is computed; buffer loads use a descriptor covering one
// (page, kv head) tile, so a page past the chunk reads zeros with no traffic.
// q is staged once through LDS (per wave) and re-read per page.
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
__device__ void matvec_wave(const DecodeParams& p, const WorkItem& it, char* smem) {
  using S = MvShape<D, R, BF16>;
  constexpr int NCH = S::NCH, EPC = S::EPC, DPL = S::DPL, LPT = S::LPT, NT = S::NT, TSTEP = S::TSTEP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % LPT, ts = lane / LPT;
  const int qi = it.id, kvh = it.kvh;
  const int tb = it.tok_begin, te = it.tok_end;
  const int npages = (te - tb + 15) >> 4;
  const int pid_lane = lane < npages ? p.pages[it.page_base + lane] : 0;

  // stage this wave's q rows (R * D elements, contiguous) in LDS
  lds_char* qs = (lds_char*)(smem + wave * S::QBYTES);
  {
    const char* qg = reinterpret_cast<const char*>(p.q) + (((int64_t)qi * p.hq + kvh * R) * D) * S::EB;
    for (int o16 = lane; o16 < S::QBYTES / 16; o16 += 64)
      *(__attribute__((address_space(3))) u32x4*)(qs + o16 * 16) = *reinterpret_cast<const u32x4*>(qg + o16 * 16);
  }
  float mref[R], mtrue[R], l[R], o[R][DPL];
  const float sc = p.scale_log2;
  const char* kpool = reinterpret_cast<const char*>(p.k);
  const char* vpool = reinterpret_cast<const char*>(p.v);

  auto load = [&](PageRegs<D, R, BF16>& b, int j) {
    // j beyond the chunk: an empty descriptor reads zeros without memory traffic
    const int pid = __builtin_amdgcn_readlane(pid_lane, j < npages ? j : 0);
    const int64_t tile = ((int64_t)pid * p.hkv + kvh) * S::TILE;
    const auto rk = make_rsrc(kpool + tile, j < npages ? S::TILE : 0u);
    const auto rv = make_rsrc(vpool + tile, j < npages ? S::TILE : 0u);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const uint32_t off = (uint32_t)(((ts + TSTEP * t) * D + (k * LPT + c) * EPC) * S::EB);
        b.k[t][k] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        b.v[t][k] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
      }
  };

  // scores of page j (log2 units, masked tokens -inf)
  auto scores = [&](const PageRegs<D, R, BF16>& b, int j, float (&s)[NT][R]) {
    // re-read q from LDS every page (an opaque offset keeps the reads in the loop)
    uint32_t qoff = (uint32_t)(c * EPC * S::EB);
    asm volatile("" : "+v"(qoff));
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
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t][h] = sum_lanes<LPT>(acc[t]);
    }
    const int tok0 = tb + j * 16 + ts;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bool ok = tok0 + TSTEP * t < te;
#pragma unroll
      for (int h = 0; h < R; ++h) s[t][h] = ok ? s[t][h] * sc : -INFINITY;
    }
  };

  // exponentials against the fixed reference max, then P.V
  auto accumulate = [&](const PageRegs<D, R, BF16>& b, const float (&s)[NT][R], bool& over) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float pr[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        mtrue[h] = fmaxf(mtrue[h], s[t][h]);
        over |= s[t][h] > mref[h] + kSlack;
        pr[t] = fast_exp2(s[t][h] - mref[h]);  // exp2(-inf) = 0 for masked tokens
        l[h] += pr[t];
      }
      if constexpr (BF16) {
#pragma unroll
        for (int t = 0; t < NT; t += 2) {
          const uint32_t pp = pack_bf16(pr[t], pr[t + 1]);
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
  bool fixed_ref = false;
  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
    }
    bool over = false;
    PageRegs<D, R, BF16> b0, b1;
    load(b0, 0);
    load(b1, 1);
    {
      float s[NT][R];
      scores(b0, 0, s);
      if (!fixed_ref) {
#pragma unroll
        for (int h = 0; h < R; ++h) {
          float mx = s[0][h];
#pragma unroll
          for (int t = 1; t < NT; ++t) mx = fmaxf(mx, s[t][h]);
          mx = fmaxf(mx, xor8(mx));
          mx = fmaxf(mx, shfl_xor(mx, 16));
          mx = fmaxf(mx, shfl_xor(mx, 32));  // page 0 always holds a valid token
          mref[h] = mx;
          mtrue[h] = -INFINITY;
        }
      }
      accumulate(b0, s, over);
    }
    load(b0, 2);
    for (int j = 1; j < npages; j += 2) {  // a page past the end is all masked zeros
      float s1[NT][R];
      scores(b1, j, s1);
      accumulate(b1, s1, over);
      load(b1, j + 2);
      float s2[NT][R];
      scores(b0, j + 1, s2);
      accumulate(b0, s2, over);
      load(b0, j + 3);
    }
    if (!__builtin_amdgcn_ballot_w64(over)) break;
    // rare: redo with the exact per-head maximum of this chunk
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mx = mtrue[h];
      mx = fmaxf(mx, xor8(mx));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      mref[h] = mx;
    }
    fixed_ref = true;
  }

  // merge the token groups (lanes with equal lane % LPT)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const bool rot = off == 8;  // lane ^ 8 within a row of 16 is row_ror:8
      const float mo = rot ? xor8(mref[h]) : shfl_xor(mref[h], off);
      const float lo = rot ? xor8(l[h]) : shfl_xor(l[h], off);
      const float mt = rot ? xor8(mtrue[h]) : shfl_xor(mtrue[h], off);
      const float M = fmaxf(mref[h], mo);
      const float a = fast_exp2(mref[h] - M), bw = fast_exp2(mo - M);
      l[h] = l[h] * a + lo * bw;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float oo = rot ? xor8(o[h][e]) : shfl_xor(o[h][e], off);
        o[h][e] = o[h][e] * a + oo * bw;
      }
      mref[h] = M;
      mtrue[h] = fmaxf(mtrue[h], mt);
    }
  }

  // lanes 0..LPT-1 write: O normalised, m (true max), l relative to it
  const int E = it.a, slot = it.b;
  if (ts == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float inv = 1.f / l[h];
      const float lt = l[h] * fast_exp2(mref[h] - mtrue[h]);
      const int64_t row = (int64_t)qi * p.hq + kvh * R + h;
      if (E == 1) {
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
          for (int q4 = 0; q4 < EPC / 4; ++q4) {
            const int e = k * EPC + q4 * 4;
            f32x4 v = {o[h][e] * inv, o[h][e + 1] * inv, o[h][e + 2] * inv, o[h][e + 3] * inv};
            store_out4(p, row * D + (k * LPT + c) * EPC + q4 * 4, v);
          }
        if (c == 0) store_ml(p, row, mtrue[h], lt);
      } else {
        const auto ro = make_rsrc(p.part_o, p.part_o_bytes);
        const uint32_t srow = (uint32_t)(slot * R + h);
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
          for (int q4 = 0; q4 < EPC / 4; ++q4) {
            const int e = k * EPC + q4 * 4;
            f32x4 v = {o[h][e] * inv, o[h][e + 1] * inv, o[h][e + 2] * inv, o[h][e + 3] * inv};
            st_coh4(ro, (srow * D + (k * LPT + c) * EPC + q4 * 4) * 4u, v);
          }
        if (c == 0) {
          const auto rm = make_rsrc(p.part_ml, p.part_ml_bytes);
          st_coh1(rm, srow * 8u, mtrue[h]);
          st_coh1(rm, srow * 8u + 4u, lt);
        }
      }
    }
  }
  if (E == 1) return;
  release_partials();
  int old = 0;
  int32_t* ctr = p.counters + (int64_t)qi * p.hkv + kvh;
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
// load unit (global_load_lds_dwordx4, no registers), double buffered: block
// b+1 is in flight while block b is computed.
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
  static constexpr int LDS_BYTES = 2 * STAGE + kMaxPrefixChunk / 16 * 4 + 128 * 4 + 16;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 layout: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }

template <int D, int R>
__device__ void prefix_mfma_tile(const DecodeParams& p, const WorkItem& it, char* smem) {
  using S = MfShape<D>;
  constexpr int KK = S::KK, NB = S::NB, NI = S::NI;
  int32_t* s_pages = reinterpret_cast<int32_t*>(smem + 2 * S::STAGE);
  int32_t* s_list = s_pages + kMaxPrefixChunk / 16;
  int* s_n = s_list + 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int g = it.id, kvh = it.kvh, rb = it.a, rc = it.b, jslot = it.kind >> 8;
  const int ntok = it.tok_end - it.tok_begin, npages = (ntok + 15) >> 4, nblocks = (ntok + 63) >> 6;
  const int32_t* mem = p.members + p.member_off[g];
  const int nslices = (rc + 15) >> 4;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q);
  const char* kp = reinterpret_cast<const char*>(p.k);
  const char* vp = reinterpret_cast<const char*>(p.v);

  for (int i = tid; i < npages; i += kThreads) s_pages[i] = p.pages[it.page_base + i];

  bool act[2];
  bf16x8 qb[2][KK];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int slice = wave + kWaves * sl;
    const int row = slice * 16 + l16;
    act[sl] = slice < nslices;
#pragma unroll
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
#pragma unroll
  for (int sl = 0; sl < 2; ++sl)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[sl][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref[2] = {kNoMax, kNoMax}, mtrue[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.f, 0.f};                  // per-lane part of the row sum of exact weights
  f32x4 rsum[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};  // row sum of rounded weights
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  const float sc = p.scale_log2;
  __syncthreads();  // s_pages ready

  // copy of one 64-token block, global -> LDS through the load unit: wave w
  // issues NI loads per tile, lane l writing 16 bytes (index maps in
  // layout.h).  Tokens past the chunk re-read its last token so every LDS row
  // stays finite (their scores are masked).
  const int64_t tile_stride = (int64_t)p.hkv * 16 * D * 2;
  auto dma = [&](int blk, int stage) {
    lds_char* kl = (lds_char*)(smem + stage * S::STAGE);
    lds_char* vl = kl + S::TILE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = mf_copy_token<D>(wave, i, lane);
      const int c = mf_copy_chunk<D>(wave, i, lane);
      int tg = blk * 64 + t;
      tg = tg < ntok ? tg : ntok - 1;
      const int64_t off = (int64_t)s_pages[tg >> 4] * tile_stride + (int64_t)kvh * 16 * D * 2 + (tg & 15) * D * 2 + c * 16;
      const int dst = mf_copy_lds<D>(wave, i, 0);  // wave-uniform base; lane l lands at +16 l
      __builtin_amdgcn_global_load_lds(kp + off, (__attribute__((address_space(3))) void*)(kl + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp + off, (__attribute__((address_space(3))) void*)(vl + dst), 16, 0, 0);
    }
  };

  dma(0, 0);
  for (int blk = 0; blk < nblocks; ++blk) {
    const int stage = blk & 1;
    if (blk + 1 < nblocks) {
      dma(blk + 1, stage ^ 1);
      __builtin_amdgcn_s_waitcnt(wait_vm(2 * NI));  // block blk landed; block blk+1 may fly
    } else {
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
    }
    __builtin_amdgcn_s_barrier();  // every wave's copy of block blk has landed
    if (act[0]) {
      const lds_char* Ks = (const lds_char*)(smem + stage * S::STAGE);
      const lds_char* Vs = Ks + S::TILE;
      // ---- S^T tiles: t = kb*2 + half covers tokens 32kb + {8*(m/4) + 4*half + m%4} ----
      f32x4 st[2][4];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int t = 0; t < 4; ++t) st[sl][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 a[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          a[kk] = *(const __attribute__((address_space(3))) bf16x8*)(Ks + mf_k_lds<D>(t, kk, lg, l16));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          st[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], qb[0][kk], st[0][t], 0, 0, 0);
          if (act[1]) st[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], qb[1][kk], st[1][t], 0, 0, 0);
        }
      }
      // ---- online softmax per row (lane's row = l16; 16 raw scores per lane) ----
      if (blk * 64 + 64 > ntok) {  // last block of the chunk: mask tokens past its end
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (blk * 64 + (t >> 1) * 32 + 8 * lg + 4 * (t & 1) + i >= ntok) st[sl][t][i] = -INFINITY;
      }
      bf16x8 pb[2][2];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        if (!act[sl]) continue;
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[sl][t][i]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        mx *= sc;  // log2 units (sc > 0 keeps the order)
        mtrue[sl] = fmaxf(mtrue[sl], mx);
        if (__builtin_amdgcn_ballot_w64(mx > mref[sl] + kLazy)) {
          const float mn = fmaxf(mref[sl], mx);
          const float alpha = fast_exp2(mref[sl] - mn);
          mref[sl] = mn;
          lrow[sl] *= alpha;
          rsum[sl] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) oacc[sl][nb] *= alpha;
        }
        const float nm = -mref[sl];
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = fast_exp2(fmaf(st[sl][kb * 2][i], sc, nm));  // exp2(-inf) = 0 when masked
            const float p1 = fast_exp2(fmaf(st[sl][kb * 2 + 1][i], sc, nm));
            ps += p0 + p1;
            v[i] = (__bf16)p0;
            v[4 + i] = (__bf16)p1;
          }
          pb[sl][kb] = v;
          // row sum of the bf16-rounded weights used in P.V, by MFMA against ones
          rsum[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, v, rsum[sl], 0, 0, 0);
        }
        lrow[sl] += ps;
      }
      // ---- O^T += V^T P^T; V^T operand through transposing LDS reads ----
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          v4i16 h[2];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            h[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(Vs + mf_v_lds<D>(kb, nb, hf, lg, l16)));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[0][kb], oacc[0][nb], 0, 0, 0);
          if (act[1]) oacc[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[1][kb], oacc[1][nb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_barrier();  // stage fully consumed before block blk+2 is copied into it
  }

  // ---- write each row's partial (or the output when the chunk is all of it) ----
  const auto ro = make_rsrc(p.part_o, p.part_o_bytes);
  const auto rm = make_rsrc(p.part_ml, p.part_ml_bytes);
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    if (!act[sl]) continue;
    float L = lrow[sl];
    L += shfl_xor(L, 16);
    L += shfl_xor(L, 32);
    const float Lr = rsum[sl][0];  // every element holds the row's sum
    const int row = (wave + kWaves * sl) * 16 + l16;
    if (row >= rc) continue;
    const int grow = rb + row;
    const int qi = mem[grow / R], hh = grow % R;
    const float inv = 1.f / Lr;  // normalise with the sum of the rounded weights used in P.V
    const float lt = L * fast_exp2(mref[sl] - mtrue[sl]);
    const int E = p.expected[qi];
    const int64_t orow = (int64_t)qi * p.hq + kvh * R + hh;
    if (E == 1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) store_out4(p, orow * D + nb * 16 + lg * 4, oacc[sl][nb] * inv);
      if (lg == 0) store_ml(p, orow, mtrue[sl], lt);
    } else {
      const uint32_t srow = (uint32_t)(((p.slot_off[qi] + jslot) * p.hkv + kvh) * R + hh);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) st_coh4(ro, (srow * D + nb * 16 + lg * 4) * 4u, oacc[sl][nb] * inv);
      if (lg == 0) {
        st_coh1(rm, srow * 8u, mtrue[sl]);
        st_coh1(rm, srow * 8u + 4u, lt);
      }
    }
  }
  // ---- arrivals of the tile's member queries; last arrivers merge ----
  release_partials();
  if (tid == 0) *s_n = 0;
  __syncthreads();
  const int nq = rc / R;
  for (int t = tid; t < nq; t += kThreads) {
    const int qi = mem[rb / R + t];
    const int E = p.expected[qi];
    if (E >= 2 && arrive_counter(p.counters + (int64_t)qi * p.hkv + kvh) == E - 1) s_list[atomicAdd(s_n, 1)] = qi;
  }
  __syncthreads();
  const int nl = *s_n;
  for (int t = wave; t < nl; t += kWaves) {
    merge_wave<D, R>(p, s_list[t], kvh);
    if (lane == 0) reset_counter(p.counters + (int64_t)s_list[t] * p.hkv + kvh);
  }
}

// Empty partial (0, -inf, 0) of every head of a query the plan does not
// cover (PREFIX_ONLY / DISTINCT_ONLY plans); one wave.
template <int D>
__device__ void empty_wave(const DecodeParams& p, const WorkItem& it) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)it.id * p.hq;
  for (int el = lane * 4; el < p.hq * D; el += 256) store_out4(p, base * D + el, f32x4{0.f, 0.f, 0.f, 0.f});
  for (int h = lane; h < p.hq; h += 64) {
    if (p.out_m) p.out_m[base + h] = -INFINITY;
    if (p.out_l) p.out_l[base + h] = 0.f;
  }
}

template <int D, int R, bool BF16>
struct Lds {
  static constexpr int MV = kWaves * MvShape<D, R, BF16>::QBYTES;
  static constexpr int MF = BF16 ? MfShape<D>::LDS_BYTES : 0;
  static constexpr int BYTES = MV > MF ? MV : MF;
};

template <int D, int R, bool BF16>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char smem[Lds<D, R, BF16>::BYTES];
  const WorkItem* unit = p.items + (int64_t)blockIdx.x * kUnitItems;
  const int kind0 = unit[0].kind & 0xff;
  if (kind0 == ITEM_PREFIX_MFMA) {
    if constexpr (BF16) prefix_mfma_tile<D, R>(p, unit[0], smem);
    return;
  }
  const WorkItem it = unit[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
  const int kind = it.kind & 0xff;
  if (kind == ITEM_MATVEC)
    matvec_wave<D, R, BF16>(p, it, smem);
  else if (kind == ITEM_EMPTY)
    empty_wave<D>(p, it);
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
