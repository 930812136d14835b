// Host check of the MFMA prefix tile's LDS index maps (layout.h): every lane,
// wave and load of the copy stays inside the tile and writes each (token,
// chunk) exactly once; every operand read stays inside the tile and finds the
// (token, chunk) the MFMA layout expects.  (Bank conflicts are not modelled
// here: the XOR key was chosen by timing the reads on the hardware.)  Exit
// status 0 = ok.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "layout.h"

using namespace psa;

static int failures = 0;
#define CHECK(c, ...)                  \
  do {                                 \
    if (!(c)) {                        \
      std::printf(__VA_ARGS__);        \
      std::printf("\n");               \
      if (++failures > 20) std::exit(1); \
    }                                  \
  } while (0)

template <int D>
void check() {
  using L = MfLayout<D>;
  // copy: where each (token, logical chunk) lands
  std::vector<int> at(64 * L::CPT, -1);
  for (int w = 0; w < L::WAVES; ++w)
    for (int i = 0; i < L::NI; ++i)
      for (int lane = 0; lane < 64; ++lane) {
        const int t = mf_copy_token<D>(w, i, lane);
        const int c = mf_copy_chunk<D>(w, i, lane);
        const int off = mf_copy_lds<D>(w, i, lane);
        CHECK(t >= 0 && t < 64, "D=%d copy token %d out of the block", D, t);
        CHECK(c >= 0 && c < L::CPT, "D=%d copy chunk %d out of the row", D, c);
        CHECK(off >= 0 && off + 16 <= L::TILE, "D=%d copy LDS offset %d out of the tile", D, off);
        CHECK(off == t * L::ROW + ((c ^ kswz<D>(t)) << 4), "D=%d copy lands off its swizzled slot", D);
        CHECK(at[t * L::CPT + c] < 0, "D=%d (token %d, chunk %d) copied twice", D, t, c);
        at[t * L::CPT + c] = off;
      }
  for (int x = 0; x < 64 * L::CPT; ++x) CHECK(at[x] >= 0, "D=%d (token %d, chunk %d) never copied", D, x / L::CPT, x % L::CPT);

  // K operand reads: 16 tokens of a tile, one logical chunk per lane group
  for (int t = 0; t < 4; ++t)
    for (int kk = 0; kk < D / 32; ++kk)
      for (int lg = 0; lg < 4; ++lg)
        for (int l16 = 0; l16 < 16; ++l16) {
          const int tok = mf_k_token<D>(t, l16);
          const int off = mf_k_lds<D>(t, kk, lg, l16);
          CHECK(off >= 0 && off + 16 <= L::TILE, "D=%d K read out of the tile", D);
          CHECK(off == at[tok * L::CPT + kk * 4 + lg], "D=%d K read misses its chunk", D);
          CHECK(off == mf_k_base<D>(kk, lg, l16) + mf_k_step<D>(t), "D=%d K read is not base + step", D);
        }
  // V^T reads: each lane's 8 bytes are 4 dims of one token; pass = 32 lanes
  for (int kb = 0; kb < 2; ++kb)
    for (int nb = 0; nb < D / 16; ++nb)
      for (int hf = 0; hf < 2; ++hf)
        for (int lane = 0; lane < 64; ++lane) {
          const int lg = lane >> 4, l16 = lane & 15;
          const int tok = mf_v_token<D>(kb, hf, lg, l16);
          const int off = mf_v_lds<D>(kb, nb, hf, lg, l16);
          const int cb = nb * 32 + (l16 & 3) * 8;
          CHECK(tok >= 0 && tok < 64, "D=%d V token out of the block", D);
          CHECK(off >= 0 && off + 8 <= L::TILE && off % 8 == 0, "D=%d V read out of the tile", D);
          CHECK(off - (cb & 15) == at[tok * L::CPT + (cb >> 4)], "D=%d V read misses its chunk", D);
          CHECK(off == mf_v_base<D>(nb, lg, l16) + mf_v_step<D>(kb, hf), "D=%d V read is not base + step", D);
        }
}

int main() {
  check<128>();
  check<64>();
  if (failures) {
    std::printf("layout check: %d failures\n", failures);
    return 1;
  }
  std::printf("layout check: ok\n");
  return 0;
}
