// Host-side check of the grouped GEMM's LDS maps (moe_expert_layer_router_amd/
// csrc/lds_layout.h): where the buffer->LDS DMA puts each 16-byte chunk of a
// tile, which logical elements the MFMA fragment reads then receive, and how
// each read phase falls on the 64 LDS banks.  Built with g++ by
// tests/test_lds_layout_cpu.py; prints one line per failed check and exits 1.
//
// What the reads must deliver (the 32x32x16 bf16 MFMA operand layout): lane l
// of a 32-row (or 32-column) block holds row (column) l % 32 and the eight
// consecutive k values 8 (l / 32) .. + 7 of the k16 sub-step.  Both ring
// depths are checked: K steps of 32 (64-byte K-contiguous rows, 32-row MN
// tiles) and K blocks of 64 (128-byte rows, 64-row MN tiles).
//   K-contiguous tiles ([rows][BKX] bf16): one ds_read_b128 per fragment.
//   MN-contiguous tiles ([BKX k][W] bf16): two ds_read_b64_tr_b16, k and k + 4;
//   within each 16-lane group lane i supplies the address of row kb + i / 4,
//   columns c0 + 4 (i % 4) .. + 3, and lane j of the group receives the four k
//   values of column c0 + j.
// Banks: 64 banks of 4 bytes; a 16-byte read is served 16 lanes at a time, an
// 8-byte read 32 lanes at a time (256 bytes per phase either way).
#include <stdint.h>
#include <stdio.h>

#include <set>
#include <utility>
#include <vector>

#include "lds_layout.h"

using namespace moe;

static int failures = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      ++failures;                        \
      if (failures < 40) {               \
        printf("FAIL: " __VA_ARGS__);    \
        printf("\n");                    \
      }                                  \
    }                                    \
  } while (0)

// ---------------------------------------------------------------- KC tiles
// rows: tile rows (BM or BN); N: DMA instructions per wave; BKX: row length.
template <int N, int BKX>
static void check_kc(int rows, const char* what) {
  constexpr int ch = BKX / 8;  // 16-byte chunks per row
  const int chunks = rows * ch;
  CHECK(4 * N * 64 == chunks, "%s: 4 waves x %d DMA x 64 lanes != %d chunks", what, N, chunks);
  std::vector<std::pair<int, int>> content(chunks, {-1, -1});  // LDS chunk -> (row, logical chunk)
  std::set<std::pair<int, int>> seen;
  for (int w = 0; w < 4; ++w)
    for (int u = 0; u < N; ++u) {
      std::set<int> lines;  // rows (global 128-byte lines) one instruction touches
      for (int l = 0; l < 64; ++l) {
        int r, c;
        kc_rows<N, BKX>(w, l, u, r, c);
        const int p = (w * N + u) * 64 + l;  // the DMA writes lds + 16 * lane
        CHECK(r >= 0 && r < rows && c >= 0 && c < ch, "%s: DMA chunk %d -> (%d, %d) outside", what, p, r, c);
        content[p] = {r, c};
        CHECK(seen.insert({r, c}).second, "%s: logical chunk (%d, %d) loaded twice", what, r, c);
        // the element index kc_idx names is where that logical chunk sits
        CHECK(kc_idx<BKX>(r, c) == p * 8, "%s: kc_idx(%d, %d) = %d, DMA put it at %d", what, r, c,
              kc_idx<BKX>(r, c), p * 8);
        // a row's BKX * 2 bytes of one step start at a multiple of BKX * 2
        // (<= 128) in memory, so they lie in one 128-byte line
        lines.insert(r);
      }
      // 1 KiB per instruction: 16 half lines (BKX = 32) or 8 whole lines (64)
      CHECK((int)lines.size() == 1024 / (BKX * 2), "%s: instruction %d of wave %d touches %zu rows", what, u, w,
            lines.size());
    }
  CHECK((int)seen.size() == chunks, "%s: %zu of %d chunks loaded", what, seen.size(), chunks);
  // fragment reads: every 32-row block, every k16 sub-step
  for (int blk = 0; blk < rows / 32; ++blk)
    for (int s = 0; s < BKX / 16; ++s) {
      std::vector<int> addr(64);
      for (int l = 0; l < 64; ++l) {
        const uint32_t a = (uint32_t)(blk * 32 * BKX * 2) + kc_lane_offset<BKX>(l, s);
        addr[l] = (int)a;
        CHECK(a % 16 == 0, "%s: unaligned fragment read", what);
        const std::pair<int, int> want = {blk * 32 + (l & 31), 2 * s + (l >> 5)};
        CHECK(content[a / 16] == want, "%s: block %d sub-step %d lane %d reads (%d, %d), wants (%d, %d)", what,
              blk, s, l, content[a / 16].first, content[a / 16].second, want.first, want.second);
      }
      for (int ph = 0; ph < 4; ++ph) {  // 16 lanes x 16 bytes per phase
        std::set<int> groups;
        for (int l = 16 * ph; l < 16 * ph + 16; ++l) groups.insert((addr[l] / 16) % 16);
        CHECK(groups.size() == 16, "%s: block %d sub-step %d phase %d: %zu of 16 bank groups", what, blk, s, ph,
              groups.size());
      }
    }
}

// ---------------------------------------------------------------- MC tiles
template <int N, int W, int BKX>
static void check_mc(const char* what) {
  constexpr int cpr = W / 8;  // 16-byte chunks per k row
  const int chunks = BKX * cpr;
  CHECK(4 * N * 64 == chunks, "%s: 4 waves x %d DMA x 64 lanes != %d chunks", what, N, chunks);
  std::vector<std::pair<int, int>> content(chunks, {-1, -1});  // LDS chunk -> (k, logical chunk)
  std::set<std::pair<int, int>> seen;
  for (int w = 0; w < 4; ++w)
    for (int u = 0; u < N; ++u)
      for (int l = 0; l < 64; ++l) {
        int k, c;
        mc_rows<N, W>(w, l, u, k, c);
        const int p = (w * N + u) * 64 + l;
        CHECK(k >= 0 && k < BKX && c >= 0 && c < cpr, "%s: DMA chunk %d -> (%d, %d) outside", what, p, k, c);
        CHECK(p / cpr == k, "%s: chunk %d is not in row %d", what, p, k);
        content[p] = {k, c};
        CHECK(seen.insert({k, c}).second, "%s: logical chunk (%d, %d) loaded twice", what, k, c);
      }
  CHECK((int)seen.size() == chunks, "%s: %zu of %d chunks loaded", what, seen.size(), chunks);
  // logical (k, column) of the bf16 element at byte address a of the slot
  auto element = [&](uint32_t a, int& k, int& col) {
    const int e = (int)(a / 2);
    k = e / W;
    const int lds_chunk = (e % W) / 8;
    col = 8 * content[k * cpr + lds_chunk].second + (e % 8);
    CHECK(content[k * cpr + lds_chunk].first == k, "%s: chunk holds another row", what);
  };
  for (int M = 0; M < W / 32; ++M)
    for (int s = 0; s < BKX / 16; ++s)
      for (int half = 0; half < 2; ++half) {  // the read of k .. k+3, then k+4 .. k+7
        std::vector<uint32_t> addr(64);
        for (int l = 0; l < 64; ++l) {
          const uint32_t a = mc_lane_offset<W>(l, M) + 2u * (16 * s * W) + (uint32_t)(half * 8 * W);
          addr[l] = a;
          CHECK(a % 8 == 0, "%s: unaligned transposing read", what);
          const int g = l >> 4, i = l & 15;
          const int kb = 16 * s + 8 * (g >> 1) + 4 * half;  // the k rows group g must deliver
          const int c0 = 32 * M + 16 * (g & 1);              // its 16 columns
          for (int q = 0; q < 4; ++q) {                      // the 4 bf16 of the lane's 8 bytes
            int k, col;
            element(a + 2 * q, k, col);
            CHECK(k == kb + i / 4 && col == c0 + 4 * (i % 4) + q,
                  "%s: M %d s %d half %d lane %d element %d at (%d, %d), wants (%d, %d)", what, M, s, half, l, q,
                  k, col, kb + i / 4, c0 + 4 * (i % 4) + q);
          }
        }
        for (int ph = 0; ph < 2; ++ph) {  // 32 lanes x 8 bytes per phase
          std::set<int> banks;
          for (int l = 32 * ph; l < 32 * ph + 32; ++l) {
            banks.insert((addr[l] / 4) % 64);
            banks.insert((addr[l] / 4 + 1) % 64);
          }
          CHECK(banks.size() == 64, "%s: M %d s %d half %d phase %d: %zu of 64 banks", what, M, s, half, ph,
                banks.size());
        }
      }
}

// ------------------------------------------------------- epilogue staging
static void check_stage() {
  std::set<int> seen;
  for (int r = 0; r < 16; ++r)
    for (int c = 0; c < 128; ++c) {
      const int i = stage_idx(r, c);
      CHECK(i >= 0 && i < 2048 && seen.insert(i).second, "stage_idx(%d, %d) = %d repeats or leaves the area", r, c,
            i);
      if (c % 4 == 0) CHECK(stage_idx(r, c + 3) == i + 3, "stage_idx splits the float4 at (%d, %d)", r, c);
    }
  // an MFMA output register q of 64 lanes: rows 4 (l / 32) + (q & 3) (+ 8 (q / 4)),
  // column 32 ni + l % 32 -> the two row halves of a write land on different banks
  for (int q = 0; q < 8; ++q)
    for (int ni = 0; ni < 4; ++ni) {
      std::set<int> banks;
      for (int l = 0; l < 64; ++l) {
        const int r = 8 * (q >> 2) + 4 * (l >> 5) + (q & 3);
        banks.insert(stage_idx(r, ni * 32 + (l & 31)) % 64);
      }
      CHECK(banks.size() == 64, "staging write q %d ni %d: %zu of 64 banks", q, ni, banks.size());
    }
}

int main() {
  // K-contiguous, K step 32: A of the 256-row and 128-row tiles (4 and 2 DMA
  // per wave), B of 256 columns (4 DMA per wave)
  check_kc<4, 32>(256, "KC 256 rows");
  check_kc<2, 32>(128, "KC 128 rows");
  // K-contiguous, K block 64: 256 rows or columns (8 DMA per wave)
  check_kc<8, 64>(256, "KC2 256 rows");
  // MN-contiguous: the 256-wide B tile and the weight gradients' A tiles
  check_mc<4, 256, 32>("MC width 256");
  check_mc<2, 128, 32>("MC width 128");
  // MN-contiguous, K block 64: the data gradients' 256-wide B tile
  check_mc<8, 256, 64>("MC2 width 256");
  check_stage();
  if (failures) {
    printf("%d failed checks\n", failures);
    return 1;
  }
  printf("all LDS maps consistent\n");
  return 0;
}
