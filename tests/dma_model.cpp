// Host model of the prefill GEMMs' global -> LDS DMA offsets.
//
// The kernels in gemm.hip compute every DMA's buffer offset with the
// functions of csrc/gemm_dma.h; this program calls the same functions for
// every wave, lane, DMA index and k slice a launch issues, over ragged
// shapes, and checks, per operand tile:
//  * the offset is either a whole 16-byte piece inside the descriptor's
//    range (rows of the tile * row pitch) or at / past the range end, so the
//    range check zero-fills it (no load straddles the end, none wraps);
//  * an in-range offset reads exactly the piece its LDS slot must hold:
//    row r of the tile (r below the tile's row count), k bytes kofs + 16p,
//    with p the swizzled piece of that slot, inside the row;
//  * every slot that must hold padding (a row past the tile's rows, a piece
//    past the row's end, a k slice that does not exist) gets an
//    out-of-range offset, i.e. zeros;
//  * offsets stay below 2^31.
// Prints one summary line; exit status 0 when every check passes.
#include "../gram_memory_layer_engram_amd/csrc/gemm_dma.h"

#include <cstdio>
#include <cstdint>
#include <vector>

namespace {

long long g_checks = 0;
int g_fail = 0;

void fail(const char* what, int total, int K, int row0, int wave, int lane, int i, uint32_t kofs, uint32_t v) {
  if (g_fail < 20)
    std::printf("FAIL %s: rows %d K %d tile row %d wave %d lane %d dma %d kofs %u voffset %u\n", what, total, K,
                row0, wave, lane, i, kofs, v);
  ++g_fail;
}

// One operand of a GEMM: `total` rows of `row_bytes`, tiles of 256 rows,
// k slices of 128 bytes (nk of them), the ktail form when the pitch is not
// a multiple of 128.
void check_operand(int total, int K, uint32_t row_bytes, int nk, bool ktail) {
  const uint32_t oob = 256u * row_bytes;
  std::vector<uint32_t> kofs_list;
  for (int d = 0; d < nk; ++d) kofs_list.push_back((uint32_t)d * engram::dma::kRowBytes);
  kofs_list.push_back(oob);
  for (int row0 = 0; row0 < total; row0 += 256) {
    const int rows = total - row0 < 256 ? total - row0 : 256;
    const uint64_t range = (uint64_t)rows * row_bytes;
    for (int wave = 0; wave < 4; ++wave)
      for (int lane = 0; lane < 64; ++lane) {
        const engram::dma::Lane l = engram::dma::lane_of(wave, lane, row_bytes);
        for (int i = 0; i < engram::dma::kDmaPerChunk; ++i)
          for (uint32_t kofs : kofs_list) {
            const uint32_t v = engram::dma::voffset(l, i, kofs, row_bytes, oob, ktail);
            ++g_checks;
            const int r = engram::dma::lds_row(wave, lane, i);
            const int piece = (lane & 7) ^ engram::dma::swizzle(r);
            const uint64_t kbyte = (uint64_t)kofs + 16u * (uint32_t)piece;
            const bool want_data = kofs != oob && r < rows && kbyte + 16 <= row_bytes;
            const bool inside = (uint64_t)v + 16 <= range;
            const bool outside = (uint64_t)v >= range;
            if (v >= 0x80000000u) fail("offset >= 2^31", total, K, row0, wave, lane, i, kofs, v);
            if (!inside && !outside) fail("straddles the range end", total, K, row0, wave, lane, i, kofs, v);
            if (want_data) {
              if (!inside || v != (uint32_t)r * row_bytes + (uint32_t)kbyte)
                fail("wrong piece for a data slot", total, K, row0, wave, lane, i, kofs, v);
            } else if (!outside) {
              fail("padding slot reads memory", total, K, row0, wave, lane, i, kofs, v);
            }
          }
      }
  }
}

}  // namespace

int main() {
  // bf16 GEMM: pitch 2K bytes, 64-element slices; K % 64 != 0 takes the ktail form
  const int bf16_shapes[][2] = {{1, 8},     {3, 32},    {33, 264},  {257, 72},  {300, 640},  {513, 1024},
                                {130, 160}, {40, 96},   {5, 64},    {70, 128},  {8192, 2048}, {20480, 2048},
                                {100, 520}, {767, 1000}, {256, 4096}, {1025, 8}};
  for (const auto& s : bf16_shapes) {
    const int rows = s[0], K = s[1];
    check_operand(rows, K, 2u * (uint32_t)K, (K + 63) / 64, K % 64 != 0);
  }
  // paced MXFP8 GEMM: pitch K bytes (K % 512 == 0), 128-byte slices
  const int mx_shapes[][2] = {{17, 512}, {257, 1024}, {300, 2048}, {32768, 3072}, {35840, 3072}, {20480, 2048},
                              {96, 3584}, {1, 512}};
  for (const auto& s : mx_shapes) {
    const int rows = s[0], K = s[1];
    check_operand(rows, K, (uint32_t)K, K / 128, false);
  }
  std::printf("dma model: %lld offsets checked, %d failures\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
