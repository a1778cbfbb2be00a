// Buffer offsets of the prefill GEMMs' global -> LDS DMAs (gemm.hip), in a
// form the host can evaluate too: tests/dma_model.cpp walks every DMA of a
// launch on the CPU and checks each offset against its descriptor's range.
//
// A raw buffer load (stride 0) range-checks only its vector offset plus the
// instruction offset against num_records; the scalar offset is added to the
// address after the check and is never checked. Every offset below therefore
// travels whole in the vector offset and the scalar offset is always 0, so:
//  * a DMA whose vector offset lies in [0, num_records - 16] reads 16 bytes
//    of the tile's own rows (num_records = rows in the tile * row pitch, the
//    pitch a multiple of 16);
//  * any other DMA (a row past the last row of W or x, a piece past a row's
//    end, or a k slice that does not exist, passed as `oob` >= num_records)
//    returns zeros into LDS and touches no memory.
// Offsets stay below 2^31: at most 2 * 256 rows of at most 2^21 bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {
namespace dma {

// One operand chunk of a k slice is 256 LDS rows of 128 bytes (8 pieces of
// 16). Wave w (0..3) issues 8 DMA instructions per chunk; instruction i
// (0..7) fills LDS rows 8*(w + 4i) .. +8 at lane*16 bytes of its 1 KiB, so
// lane l writes LDS row 8*(w + 4i) + l/8, position l%8. Position p of LDS
// row r holds global piece p ^ ((r >> 1) & 7), which makes the 32-row
// fragment reads conflict-free. That XOR does not depend on i: rows 32*i
// apart agree in bits 1..3.
constexpr int kRowBytes = 128;
constexpr int kDmaPerChunk = 8;

struct Lane {
  uint32_t pofs;   // byte offset of the lane's global piece inside its row's slice
  uint32_t vrow;   // vector offset of the lane's piece for DMA 0 at k offset 0
};

__host__ __device__ inline int swizzle(int row) { return (row >> 1) & 7; }

__host__ __device__ inline int lds_row(int wave, int lane, int i) { return 8 * (wave + 4 * i) + (lane >> 3); }

__host__ __device__ inline Lane lane_of(int wave, int lane, uint32_t row_bytes) {
  const int piece = (lane & 7) ^ swizzle(lds_row(wave, lane, 0));
  Lane l;
  l.pofs = (uint32_t)piece * 16u;
  l.vrow = (uint32_t)lds_row(wave, lane, 0) * row_bytes + l.pofs;
  return l;
}

// Vector offset of DMA i for the k slice at byte offset kofs of each row
// (kofs = oob for a slice that does not exist). ktail: the row pitch is not
// a multiple of the slice (K % 64 != 0 in bf16), so a piece at or past the
// row's end is sent to oob as well.
__host__ __device__ inline uint32_t voffset(const Lane& l, int i, uint32_t kofs, uint32_t row_bytes,
                                            uint32_t oob, bool ktail) {
  if (ktail && kofs + l.pofs >= row_bytes) return oob;
  return l.vrow + (uint32_t)(32 * i) * row_bytes + kofs;
}

}  // namespace dma
}  // namespace engram
