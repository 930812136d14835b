// Index maps of the MFMA prefix tile's LDS staging, shared by the kernel and
// by a host-side checker (layout_check.cpp) that enumerates every lane.
//
// One 64-token block of K (or V) for one kv head is a [64 tokens][D] bf16
// tile in LDS, rows of D*2 bytes.  Each row's 16-byte chunks are XOR-swizzled
// by a key of the token: physical chunk = logical chunk ^ kswz(t).
//
// Copy (global -> LDS, one 16-byte load per lane): wave w issues NI loads per
// tile; load i fills LDS bytes [(w*NI + i) KiB, +1 KiB) of the tile, lane l
// writing 16 bytes at l*16.  That lane therefore fetches token
// (w*NI + i)*TPI + l/CPT and logical chunk (l % CPT) ^ kswz(token).
//
// Reads: the K operand of S^T = K Q^T (tile t = kb*2+half, k-step kk) reads
// token 32kb + 8*(l16/4) + 4*half + l16%4, logical chunk kk*4 + lg.  The V^T
// operand of O^T = V^T P^T reads, with ds_read_b64_tr_b16, 8 bytes at token
// 32kb + 8lg + 4hf + l16/4 and byte column nb*32 + (l16%4)*8.
#pragma once

#ifndef __HIPCC__
#define PSA_HD inline
#else
#define PSA_HD __host__ __device__ __forceinline__
#endif

namespace psa {

template <int D>
struct MfLayout {
  static constexpr int CPT = D / 8;                 // 16-byte chunks per token row
  static constexpr int ROW = D * 2;                 // bytes per token row
  static constexpr int TILE = 64 * ROW;             // one 64-token tile (bytes)
  static constexpr int TPI = 1024 / ROW;            // tokens per 1 KiB load
  static constexpr int WAVES = 4;
  static constexpr int NI = TILE / 1024 / WAVES;    // 1 KiB loads per wave per tile
  static_assert(NI * WAVES * 1024 == TILE, "tile must split into whole KiB loads per wave");
};

// chunk XOR key of token t (t within a 64-token block).  Any key that is a
// function of the token keeps the copy and the reads consistent; these were
// chosen by timing keys made of token bits on gfx950, two workgroups per CU
// (where the LDS, not the issue, bounds the reads):
// - D 128: token bits 0, 1, 3 in key bits 1, 2, 3 (key bit 0 stays 0).  A
//   K operand read (ds_read_b128) is served 8 lanes at a time, whose 8
//   tokens differ in bits 0, 1, 3: their chunks must differ.  A transposing
//   V read (ds_read_b64_tr_b16) is served 32 lanes at a time: 8 tokens (bits
//   0, 1, 3 again) x the two chunks 2nb and 2nb + 1, which fill all 64
//   banks only if key bit 0 is the same for all 8 tokens.  The previous key
//   (bits 0, 1, 3, 4 in key bits 0..3) made every V read take two passes
//   (the bank-conflict counter's half of the V reads' LDS cycles; 26.9
//   against 18.3 cycles per read and wave), and e.g. bits 4, 2, 0, 1 make
//   the K reads 1.8x slower.
// - D 64 (rows of 128 bytes, two tokens per bank line, token bit 0 picks
//   the line's half): token bits 0, 1, 3.
// The key of a read's token depends only on the lane (bits 0, 1 and 3 of the
// token come from the lane, bits 2 and 5 from the read's step), so a read is
// a per-lane base plus a step the kernel adds as an immediate.
template <int D>
PSA_HD int kswz(int t) {
  if (D == 128) return ((t & 3) << 1) | (((t >> 3) & 1) << 3);
  return (t & 3) | (((t >> 3) & 1) << 2);
}

// copy: token and logical chunk fetched by (wave, load i, lane); LDS byte offset written
template <int D>
PSA_HD int mf_copy_token(int wave, int i, int lane) {
  return (wave * MfLayout<D>::NI + i) * MfLayout<D>::TPI + lane / MfLayout<D>::CPT;
}
template <int D>
PSA_HD int mf_copy_chunk(int wave, int i, int lane) {
  return (lane % MfLayout<D>::CPT) ^ kswz<D>(mf_copy_token<D>(wave, i, lane));
}
template <int D>
PSA_HD int mf_copy_lds(int wave, int i, int lane) {
  return (wave * MfLayout<D>::NI + i) * 1024 + lane * 16;
}

// K operand read: 16 bytes
template <int D>
PSA_HD int mf_k_token(int t, int l16) {
  return (t >> 1) * 32 + 8 * (l16 >> 2) + 4 * (t & 1) + (l16 & 3);
}
template <int D>
PSA_HD int mf_k_lds(int t, int kk, int lg, int l16) {
  const int tok = mf_k_token<D>(t, l16);
  return tok * MfLayout<D>::ROW + (((kk * 4 + lg) ^ kswz<D>(tok)) << 4);
}

// The key of a K operand token depends only on the lane (the token bits it
// uses come from l16), so the read of tile t is the tile-0 read plus a step
// that depends on t alone; likewise the V^T read of (kb, hf) is the (0, 0)
// read plus a step.  The kernel holds the per-lane bases in registers and
// adds the steps as immediates.
template <int D>
PSA_HD int mf_k_base(int kk, int lg, int l16) { return mf_k_lds<D>(0, kk, lg, l16); }
template <int D>
PSA_HD constexpr int mf_k_step(int t) { return ((t >> 1) * 32 + 4 * (t & 1)) * MfLayout<D>::ROW; }

// V^T operand read (ds_read_b64_tr_b16): 8 bytes
template <int D>
PSA_HD int mf_v_token(int kb, int hf, int lg, int l16) {
  return kb * 32 + 8 * lg + 4 * hf + (l16 >> 2);
}
template <int D>
PSA_HD int mf_v_lds(int kb, int nb, int hf, int lg, int l16) {
  const int tok = mf_v_token<D>(kb, hf, lg, l16);
  const int cb = nb * 32 + (l16 & 3) * 8;
  return tok * MfLayout<D>::ROW + ((((cb >> 4) ^ kswz<D>(tok)) << 4) | (cb & 15));
}

template <int D>
PSA_HD int mf_v_base(int nb, int lg, int l16) { return mf_v_lds<D>(0, nb, 0, lg, l16); }
template <int D>
PSA_HD constexpr int mf_v_step(int kb, int hf) { return (kb * 32 + 4 * hf) * MfLayout<D>::ROW; }

}  // namespace psa
